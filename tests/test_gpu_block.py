"""Block and stack parity against the float64 oracle, and determinism (GPU).

The whole forward runs through ``moss_block_forward`` / ``moss_stack_forward``
on seeded bf16 inputs; the oracle computes the same block in float64 on the
same bits with its own rotary tables.  Each output is gated by the acceptance
bar (cosine >= 0.9997 and max|err| <= 2e-2 max|ref|), both on the output and
on the block's update (output minus the joined input rows), which is the part
the block computes.
"""
import numpy as np
import pytest

from diffusion_transformer_denoiser_amd import moss, synth
from oracle import dit_block as ob

from . import gates
from . import gpu_util as G

pytestmark = pytest.mark.gpu

STRONG = 0.02 * np.sqrt(3072 / 256)  # small geometry with the D=3072 block's branch magnitudes


@pytest.fixture(scope="module", autouse=True)
def gpu():
    t = G.torch()
    assert t.cuda.is_available(), "no GPU visible"
    assert moss.moss_device_check(0) == moss.MOSS_OK, "device 0 is not gfx950"
    return t


def gpu_forward(geom, acts, wbits, workspace=None, out=None):
    """Run the block (one weight dict) or the stack (a list) on the GPU; returns the output tensor."""
    t = G.torch()
    blocks = wbits if isinstance(wbits, list) else [wbits]
    dims = G.geometry_dims(geom)
    rope = G.empty_f32(2, geom.rows, 64)
    moss.moss_rope_build(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, rope)
    if workspace is None:
        workspace = t.empty(moss.moss_workspace_bytes(dims, len(blocks)), dtype=t.uint8, device="cuda")
    if out is None:
        out = G.empty_bf16(geom.batch, geom.rows, geom.d_model)
    dev_w = [{k: G.dev(v) for k, v in w.items()} for w in blocks]
    x, txt, cond = G.dev(acts["x"]), G.dev(acts["txt"]), G.dev(acts["cond"])
    if isinstance(wbits, list):
        moss.moss_stack_forward(dims, dev_w, x, txt, acts["txt_len"], cond, rope, out, workspace)
    else:
        moss.moss_block_forward(dims, x, txt, acts["txt_len"], cond, dev_w[0], rope, out, workspace)
    G.sync()
    return out


def oracle_forward(geom, acts, wbits, rounded=False):
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    x, txt, cond = ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), ob.widen_bf16(acts["cond"])
    if isinstance(wbits, list):
        return ob.stack_forward(x, txt, acts["txt_len"], cond, (ob.weights_f64(w) for w in wbits), cos, sin,
                                geom.eps, rounded=rounded)
    return ob.block_forward(x, txt, acts["txt_len"], cond, ob.weights_f64(wbits), cos, sin, geom.eps,
                            rounded=rounded)


def check(geom, acts, got, ref, delta_bar=True):
    h0 = ob.join_rows(ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), acts["txt_len"])
    G.assert_parity("out", got, ref)
    if delta_bar:
        G.assert_parity("out - h0", got - h0, ref - h0)


def test_block_small_workload():
    """72 rows, D=256, weights N(0, 0.02): the update is ~1% of the residual, so out is
    also held to within 2 bf16 ulps of the exact result."""
    geom = synth.CONFIGS["c0"]
    G.say("block c0")
    acts = synth.make_activations(geom, 0)
    w = synth.make_block_weights(geom, 0, 0)
    got = G.host_f64(gpu_forward(geom, acts, w))
    ref = oracle_forward(geom, acts, w)
    check(geom, acts, got, ref, delta_bar=False)
    G.assert_ulps("out", got, ref, ulps=2.0, abs_floor=1e-3)


@pytest.mark.parametrize("batch,lens", [(1, None), (2, (8, 3)), (3, (0, 8, 5))])
def test_block_small_strong_branches(batch, lens):
    geom = synth.smaller(synth.CONFIGS["c0"], batch=batch, txt_len=lens or ())
    G.say(f"block c0-strong B={batch} txt_len={lens}")
    acts = synth.make_activations(geom, 1)
    w = synth.make_block_weights(geom, 1, 0, std=STRONG)
    got = G.host_f64(gpu_forward(geom, acts, w))
    ref = oracle_forward(geom, acts, w)
    check(geom, acts, got, ref)


def test_block_sharp_logits():
    """q/k gains near 4 (logits about N(0, 16)) at a ragged 150-row geometry.

    Sharp softmaxes amplify the bf16 rounding of the stored q and k (about
    2^-9 per element, so logit errors of ~0.02 and probability errors of ~2%
    on the dominant keys), a property of the bf16 storage policy rather than
    of any kernel: the oracle's own rounding-point mode sits over 2e-2 (max
    error) from its exact mode on this input
    (``test_oracle_pins.py::test_sharp_logits_storage_policy_gap``).  The bar is therefore applied against the oracle's
    rounding-point mode, which stores q, k and every other intermediate in
    bf16 as the GPU path does; the exact-mode cosine is still checked.
    """
    geom, acts, w = gates.sharp_logits_case()
    G.say("block sharp")
    got = G.host_f64(gpu_forward(geom, acts, w))
    check(geom, acts, got, oracle_forward(geom, acts, w, rounded=True))
    G.assert_parity("out (exact oracle)", got, oracle_forward(geom, acts, w), rel_max=5e-2)


# c1-c3, and the larger pictures of the CUDA port page's served-picture table
# (5120, 5632 and 6144 image rows; the last is the one its server refused for memory)
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "p1280", "p1408", "p1536"])
def test_block_full_size(name):
    geom = synth.CONFIGS[name]
    G.say(f"block {name}: {geom.n_txt}+{geom.n_img} rows, D={geom.d_model}")
    acts = synth.make_activations(geom, 0)
    w = synth.make_block_weights(geom, 0, 0)
    got = G.host_f64(gpu_forward(geom, acts, w))
    G.say("  oracle ...")
    ref = oracle_forward(geom, acts, w)
    check(geom, acts, got, ref)


def test_block_zero_gates_is_identity():
    """gate1 = gate2 = 0: the output is the joined input, bit for bit."""
    geom = synth.smaller(synth.CONFIGS["c1"], batch=2, txt_len=(34, 10))
    G.say("block zero gates")
    acts = synth.make_activations(geom, 3)
    w = synth.make_block_weights(geom, 3, 0)
    d = geom.d_model
    w["w_mod"][2 * d:3 * d] = 0
    w["w_mod"][5 * d:6 * d] = 0
    got = G.host_f64(gpu_forward(geom, acts, w))
    np.testing.assert_array_equal(got, ob.join_rows(ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]),
                                                    acts["txt_len"]))


def test_block_repeats_are_byte_identical():
    """The same call three times, with a different call between, gives identical bytes."""
    t = G.torch()
    geom = synth.CONFIGS["c2"]
    other = synth.CONFIGS["c1"]
    G.say("determinism c2")
    acts = synth.make_activations(geom, 0)
    w = synth.make_block_weights(geom, 0, 0)
    dims = G.geometry_dims(geom)
    ws = t.empty(moss.moss_workspace_bytes(dims, 1), dtype=t.uint8, device="cuda")
    outs = []
    for i in range(3):
        outs.append(G.host_bits(gpu_forward(geom, acts, w, workspace=ws)))
        if i == 0:
            gpu_forward(other, synth.make_activations(other, 5), synth.make_block_weights(other, 5, 0))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_block_reads_no_unwritten_scratch():
    """A workspace full of NaN bytes (0xFF) before the call gives the same output bytes as a
    zeroed one: no kernel reads scratch the call has not written first."""
    t = G.torch()
    geom = synth.smaller(synth.CONFIGS["c0"], batch=2, txt_len=(8, 3))
    G.say("workspace poisoned with NaN bytes")
    acts = synth.make_activations(geom, 14)
    w = synth.make_block_weights(geom, 14, 0, std=STRONG)
    dims = G.geometry_dims(geom)
    ws = t.empty(moss.moss_workspace_bytes(dims, 1), dtype=t.uint8, device="cuda")
    ws.fill_(0)
    clean = G.host_bits(gpu_forward(geom, acts, w, workspace=ws))
    ws.fill_(255)
    poisoned = G.host_bits(gpu_forward(geom, acts, w, workspace=ws))
    np.testing.assert_array_equal(poisoned, clean)


def test_stack_small():
    geom = synth.smaller(synth.CONFIGS["c0"], batch=2, txt_len=(8, 2))
    G.say("stack c0-strong x3")
    acts = synth.make_activations(geom, 4)
    ws = [synth.make_block_weights(geom, 4, i, std=STRONG) for i in range(3)]
    got = G.host_f64(gpu_forward(geom, acts, ws))
    check(geom, acts, got, oracle_forward(geom, acts, ws))


def test_stack_guidance_pair_two_blocks():
    """Two blocks at the full guidance-pair geometry (4096+34 rows, items with 34 and 10 text rows)."""
    geom = synth.CONFIGS["c4"]
    G.say("stack c4 x2")
    acts = synth.make_activations(geom, 0)
    ws = [synth.make_block_weights(geom, 0, i) for i in range(2)]
    got = G.host_f64(gpu_forward(geom, acts, ws))
    G.say("  oracle ...")
    check(geom, acts, got, oracle_forward(geom, acts, ws))
