"""The acceptance checks of the GPU parity tests, with the inputs and references they use.

The GPU tests apply these checks to what the HIP path returns; the CPU tests in
``test_gate_sensitivity.py`` apply the same checks, at the same shapes and
tolerances, to the outputs of planted mistakes in the oracle (a dropped rounding
point, a rotary pair turned the wrong way, a key mask off by one, a dropped gate)
and require each to be rejected, as the pages' planted controls must come out
red (the encoder page, PR #1512, "Receipt").  Nothing here touches a GPU.
"""
from __future__ import annotations

import numpy as np

from diffusion_transformer_denoiser_amd import synth
from oracle import dit_block as ob

from . import gpu_util as G

# ---- a3 + a4: the QKV projection with the q/k norm, rotary and packing -------------------------

QKV_PACK_SHAPES = [
    (1, 8, 8, 8, 2),      # one 128-row tile of rows, two heads
    (2, 34, 8, 12, 3),    # items that straddle row tiles; D = 384: a tile spans q and k columns
    (1, 34, 64, 64, 24),  # the 4096+34-row QKV (column split: the last 6 column tiles run as 128-row tiles)
    (2, 34, 64, 64, 24),  # the guidance pair's QKV, 2 x 4130 rows, as each block of the stack runs it
]


def qkv_pack_case(batch, n_txt, gh, gw, heads):
    """Seeded inputs of the fused QKV test: activations a, W_qkv, the two gains; rotary tables;
    the rows checked (all of them, or a sample at the full size)."""
    rows = n_txt + gh * gw
    d = heads * 128
    case = dict(batch=batch, rows=rows, heads=heads, d=d, n_txt=n_txt, gh=gh, gw=gw)
    case["a"] = synth.make_tensor(10, 0, (batch * rows, d))
    case["w"] = synth.make_tensor(10, 1, (3 * d, d), std=0.02)
    case["gq"] = synth.normal_bf16(10, (0, 50), (128,), 0.02, offset=1.0)
    case["gk"] = synth.normal_bf16(10, (0, 51), (128,), 0.02, offset=1.0)
    case["cos"], case["sin"] = ob.rope_tables(n_txt, gh, gw, 10000.0, 128)
    case["sel"] = np.arange(rows) if rows <= 1100 else np.unique(
        np.r_[0:40, rows - 40:rows, np.linspace(0, rows - 1, 120).astype(int)])
    return case


def qkv_pack_reference(case, b, round_projection=True, qk_norm_rope=None):
    """The oracle's a4 on the bf16-rounded projection for item b at the checked rows:
    (q, k, v), each [H, len(sel), 128].  The keyword hooks let a CPU test plant a mistake."""
    sel, rows, d, heads = case["sel"], case["rows"], case["d"], case["heads"]
    arows = ob.widen_bf16(case["a"].reshape(case["batch"], rows, d)[b][sel])
    proj = arows @ ob.widen_bf16(case["w"]).T
    if round_projection:
        proj = ob.round_bf16(proj)
    qkv = proj.reshape(len(sel), 3, heads, 128).transpose(1, 2, 0, 3)
    fn = qk_norm_rope or ob.qk_norm_rope
    rq, rk = fn(qkv[0], qkv[1], ob.widen_bf16(case["gq"]), ob.widen_bf16(case["gk"]), case["cos"][sel],
                case["sin"][sel], 1e-6)
    return rq, rk, qkv[2]


def check_qkv_pack(name, got, ref):
    """q or k: within 2 bf16 ulps + 8e-3 everywhere, and 99.9% of values within one ulp.

    The projection's fp32 sum can round to the other bf16 neighbour of the exact sum (as the
    unfused GEMM's output can); such an input flip moves a normed value by about 2^-8 of the
    row scale (about 1), hence the 8e-3 floor; nearly all values must agree to one ulp."""
    G.assert_ulps(name, got, ref, ulps=2.0, abs_floor=8e-3)
    tight = np.abs(got - ref) <= G.bf16_ulp(ref) + 2e-5
    assert tight.mean() >= 0.999, f"{name}: {100 * (1 - tight.mean()):.3f}% beyond one ulp"


# ---- a5 attention ------------------------------------------------------------------------------

def attention_inputs(batch, heads, rows, seed, q_scale=1.0, n_txt=0, lens=None, pad_dominant=False):
    """q, k, v bits [B, H, rows, 128].  With pad_dominant, every query gets +1 in each dimension
    and each pad key (text rows at or past the item's length) is the all-ones row with values of
    4: its logit is about 11 against about N(0, 2) for the others, so one pad key let through
    takes most of a query's weight (an adversarial input for the key mask, in the manner of the
    pages' gate 4)."""
    if pad_dominant:
        q = ob.widen_bf16(synth.make_tensor(seed, 0, (batch, heads, rows, 128), std=q_scale)) + 1.0
        q = synth.f32_to_bf16_bits(q.astype(np.float32))
    else:
        q = synth.make_tensor(seed, 0, (batch, heads, rows, 128), std=q_scale)
    k = synth.make_tensor(seed, 1, (batch, heads, rows, 128))
    v = synth.make_tensor(seed, 2, (batch, heads, rows, 128), std=1.3)
    if pad_dominant:
        for b in range(batch):
            n = lens[b] if lens is not None else n_txt
            k[b, :, n:n_txt] = 0x3F80  # 1.0
            v[b, :, n:n_txt] = 0x4080  # 4.0
    return q, k, v


def attention_reference(q, k, v, n_txt, lens, key_mask=None):
    """The oracle's attention per item: [B, H, rows, 128] float64."""
    batch, rows = q.shape[0], q.shape[2]
    mask_fn = key_mask or ob.key_mask
    refs = []
    for b in range(batch):
        valid = mask_fn(n_txt, rows - n_txt, [lens[b] if lens is not None else n_txt])[0]
        refs.append(ob.attention(ob.widen_bf16(q[b]), ob.widen_bf16(k[b]), ob.widen_bf16(v[b]), valid))
    return np.stack(refs)


def check_attention(got, ref):
    G.assert_parity("o", got, ref, cos_min=0.99995, rel_max=1e-2)


# ---- the block -------------------------------------------------------------------------------

def sharp_logits_case():
    """The sharp-logit block: q/k gains near 4 (logits about N(0, 16)) at a ragged 150-row
    geometry (12 text + 12 x 12 image rows, D = 384, 3 heads), branch magnitudes of the D = 3072
    block.  Returns (geometry, activation bits, weight bits)."""
    geom = synth.Geometry("sharp", 1, 6, 12, 12, 384, 3, 512)
    acts = synth.make_activations(geom, 2)
    w = synth.make_block_weights(geom, 2, 0, std=0.02 * np.sqrt(3072 / 384), gain_mean=4.0, gain_std=0.08)
    return geom, acts, w


def check_block(got, ref, h0, delta_bar=True):
    """The acceptance bar on the output and on the block's update (output minus the joined rows)."""
    G.assert_parity("out", got, ref)
    if delta_bar:
        G.assert_parity("out - h0", got - h0, ref - h0)
