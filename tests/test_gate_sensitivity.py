"""The GPU tests' checks reject planted mistakes (CPU only; no kernel is broken on a GPU).

Each case builds the inputs of one GPU test, computes that test's reference, then
computes the same step with one plausible mistake planted in the oracle (what a
faulty kernel would return), and requires the test's own check, at its own shapes
and tolerances, to fail on it: the pages' planted controls that must come out
red (the encoder page, PR #1512, "Receipt").
"""
import numpy as np
import pytest

from diffusion_transformer_denoiser_amd import synth
from oracle import dit_block as ob

from . import gates
from . import gpu_util as G


def _rotate_backwards(x, cos, sin):
    return ob.rope_rotate(x, cos, -sin)


def _rotate_half_split(x, cos, sin):
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def _qk_with_rotation(rot):
    def fn(q, k, qg, kg, cos, sin, eps, rnd=ob._ident):
        return (rnd(rot(ob.rms_normalize(q, eps) * qg, cos, sin)), rnd(rot(ob.rms_normalize(k, eps) * kg, cos, sin)))
    return fn


QKV_MISTAKES = {
    "qkv rounding point dropped": dict(round_projection=False),
    "rotary pairs turned backwards": dict(qk_norm_rope=_qk_with_rotation(_rotate_backwards)),
    "rotary pairs split in halves": dict(qk_norm_rope=_qk_with_rotation(_rotate_half_split)),
}


@pytest.mark.parametrize("shape", gates.QKV_PACK_SHAPES, ids=lambda s: f"B{s[0]}-H{s[4]}-rows{s[1] + s[2] * s[3]}")
@pytest.mark.parametrize("mistake", sorted(QKV_MISTAKES))
def test_qkv_pack_check_rejects(shape, mistake):
    case = gates.qkv_pack_case(*shape)
    failed = []
    for b in range(case["batch"]):
        rq, rk, _ = gates.qkv_pack_reference(case, b)
        mq, mk, _ = gates.qkv_pack_reference(case, b, **QKV_MISTAKES[mistake])
        for name, got, ref in (("q", ob.round_bf16(mq), rq), ("k", ob.round_bf16(mk), rk)):
            try:
                gates.check_qkv_pack(name, got, ref)
            except AssertionError:
                failed.append(name)
    assert failed, f"{mistake}: the fused-QKV check passed it"


def test_qkv_pack_check_accepts_the_reference_rounded():
    """The reference itself, stored in bf16, passes (the check is not rejecting everything)."""
    case = gates.qkv_pack_case(*gates.QKV_PACK_SHAPES[1])
    for b in range(case["batch"]):
        rq, rk, _ = gates.qkv_pack_reference(case, b)
        gates.check_qkv_pack("q", ob.round_bf16(rq), rq)
        gates.check_qkv_pack("k", ob.round_bf16(rk), rk)


_key_mask = ob.key_mask


def _mask_off_by_one(n_txt, n_img, txt_len):
    m = _key_mask(n_txt, n_img, txt_len)
    for b, n in enumerate(txt_len):
        if int(n) < n_txt:
            m[b, int(n)] = True
    return m


def _mask_other_item(batch_lens):
    def fn(n_txt, n_img, txt_len):
        # the length of the item's neighbour in the batch (the wrong index into txt_len)
        n = int(txt_len[0])
        other = batch_lens[(batch_lens.index(n) + 1) % len(batch_lens)]
        return _key_mask(n_txt, n_img, [other])
    return fn


# (case, inputs): the pad-dominant tests' inputs, and the plain guidance-pair case of test_attention
MASK_CASES = [((2, 2, 4130, 34, (34, 10)), "pad-dominant", 9), ((2, 3, 200, 150, (1, 149)), "pad-dominant", 9),
              ((2, 2, 4130, 34, (34, 10)), "plain", 7)]


@pytest.mark.parametrize("case,inputs,seed", MASK_CASES, ids=lambda c: str(c))
@pytest.mark.parametrize("mistake", ["off by one", "other item's length"])
def test_attention_check_rejects_mask_mistakes(case, inputs, seed, mistake):
    """A key mask off by one, or taken from the other item, fails the attention check."""
    batch, heads, rows, n_txt, lens = case
    q, k, v = gates.attention_inputs(batch, heads, rows, seed, 1.0, n_txt, lens, pad_dominant=inputs == "pad-dominant")
    ref = gates.attention_reference(q, k, v, n_txt, lens)
    mask = _mask_off_by_one if mistake == "off by one" else _mask_other_item(list(lens))
    got = ob.round_bf16(gates.attention_reference(q, k, v, n_txt, lens, key_mask=mask))
    with pytest.raises(AssertionError):
        gates.check_attention(got, ref)
    gates.check_attention(ob.round_bf16(ref), ref)  # and the reference stored in bf16 passes


# ---- the block bar ------------------------------------------------------------------------------

def _gated_add_no_gate(h, gate, y):
    return h + y


# A key mask off by one is not among them: in a block the pad text rows enter as zero rows, so the
# key let through is an ordinary key (one of 67 here) and moves the block output by about 0.5%,
# inside the block bar.  The attention tests above are the mask's gate, and they reject it.
BLOCK_MISTAKES = {
    "first gate dropped": ("gated_add", _gated_add_no_gate),
    "rotary pairs turned backwards": ("qk_norm_rope", _qk_with_rotation(_rotate_backwards)),
}


@pytest.mark.parametrize("mistake", sorted(BLOCK_MISTAKES))
def test_block_check_rejects(mistake, monkeypatch):
    """The block bar at the strong-branch small geometry (batch 2, 8 and 3 valid text rows)."""
    geom = synth.smaller(synth.CONFIGS["c0"], batch=2, txt_len=(8, 3))
    acts = synth.make_activations(geom, 1)
    w = ob.weights_f64(synth.make_block_weights(geom, 1, 0, std=0.02 * np.sqrt(3072 / 256)))
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    x, txt, cond = ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), ob.widen_bf16(acts["cond"])
    ref = ob.block_forward(x, txt, acts["txt_len"], cond, w, cos, sin, geom.eps)
    h0 = ob.join_rows(x, txt, acts["txt_len"])
    attr, fn = BLOCK_MISTAKES[mistake]
    monkeypatch.setattr(ob, attr, fn)
    got = ob.block_forward(x, txt, acts["txt_len"], cond, w, cos, sin, geom.eps, rounded=True)
    with pytest.raises(AssertionError):
        gates.check_block(got, ref, h0)
    monkeypatch.undo()
    gates.check_block(ob.block_forward(x, txt, acts["txt_len"], cond, w, cos, sin, geom.eps, rounded=True), ref, h0)
