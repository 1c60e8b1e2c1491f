"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

from diffusion_transformer_denoiser_amd import synth
from oracle import dit_block as ob

from . import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


def test_brute_force_c0():
    """The NumPy oracle equals the loop-only brute force on the small workload (72 rows, D=256)."""
    geom = synth.CONFIGS["c0"]
    x, txt, lens, cond, ws = P.f64_inputs(geom, seed=0)
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    got = ob.block_forward(x, txt, lens, cond, ws[0], cos, sin, geom.eps)
    ref = P._brute_block(geom, x, txt, lens, cond, ws[0])
    P._close(got, ref, 1e-12)


def test_rounded_mode_close_to_exact():
    """The bf16-rounding-point mode stays near the exact mode, step by step.

    At the small workload the block's update is about 1% of the residual, so
    the output is compared at bf16 resolution and every intermediate by
    cosine.
    """
    geom = synth.CONFIGS["c0"]
    x, txt, lens, cond, ws = P.f64_inputs(geom, seed=0)
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    a, sa = ob.block_forward(x, txt, lens, cond, ws[0], cos, sin, geom.eps, keep=True)
    b, sb = ob.block_forward(x, txt, lens, cond, ws[0], cos, sin, geom.eps, rounded=True, keep=True)
    for k in sa:
        u, v = sa[k].ravel(), sb[k].ravel()
        assert 1.0 - float(u @ v / np.linalg.norm(u) / np.linalg.norm(v)) < 5e-5, k
    assert np.max(np.abs(a - b)) <= 2.0 ** -7 * np.max(np.abs(a))
    assert not np.array_equal(a, b)


def test_acceptance_gate_catches_a_planted_row_error():
    """The block bar (cosine >= 0.9997, max|err| <= 2e-2 max|ref|) fails on an output whose
    only fault is one row off by 5%, as the pages' per-step gate must (the encoder page,
    "Receipt": a planted 5% row error fails even when repeats are identical)."""
    from . import gpu_util as G
    geom = P.tiny_geoms()[1]
    x, txt, lens, cond, ws = P.f64_inputs(geom, seed=8)
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    ref = ob.block_forward(x, txt, lens, cond, ws[0], cos, sin, geom.eps)
    G.assert_parity("unchanged", ref.copy(), ref)
    bad = ref.copy()
    row = int(np.argmax(np.abs(ref).max(axis=-1).ravel()))
    bad.reshape(-1, ref.shape[-1])[row] *= 1.05
    with pytest.raises(AssertionError):
        G.assert_parity("one row 5% off", bad, ref)


def test_sharp_logits_storage_policy_gap():
    """On the sharp-logit block's input, storing the intermediates in bf16 alone (the oracle's
    rounding-point mode, no kernel involved) moves the output more than 2e-2 of its maximum from
    the exact result, on the output and on the update: the reason that GPU test applies the bar
    against the rounding-point mode.  The cosines stay above 0.9997."""
    from . import gates
    from . import gpu_util as G
    geom, acts, w = gates.sharp_logits_case()
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    x, txt, cond = ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), ob.widen_bf16(acts["cond"])
    wf = ob.weights_f64(w)
    exact = ob.block_forward(x, txt, acts["txt_len"], cond, wf, cos, sin, geom.eps)
    rounded = ob.block_forward(x, txt, acts["txt_len"], cond, wf, cos, sin, geom.eps, rounded=True)
    h0 = ob.join_rows(x, txt, acts["txt_len"])
    assert G.max_rel(rounded, exact) >= 2e-2, G.max_rel(rounded, exact)
    assert G.max_rel(rounded - h0, exact - h0) >= 2e-2, G.max_rel(rounded - h0, exact - h0)
    assert G.cos_sim(rounded, exact) >= 0.9997 and G.cos_sim(rounded - h0, exact - h0) >= 0.9997
