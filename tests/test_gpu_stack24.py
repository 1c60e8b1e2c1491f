"""The 24-block guidance-pair stack against the float64 oracle (GPU).

Workload: 24 blocks, D = 3072, 24 heads x 128, MLP 12288, batch 2 at 4096 image
+ 34 text rows per item, the second item with 10 valid text rows.  The GPU
output is computed once per module.  Two checks:

* against the committed oracle record (``tests/golden/stack24_c4_rows.npz``,
  written by ``tests/golden/make_stack_golden.py``, which runs only the
  oracle): 16 sampled rows element by element, and every row of both items
  through its sketch (norm, and 16 fixed Gaussian projections, of the output
  and of the update out - h0);
* against the oracle run here, on the host's cores, on every element of both
  items (about 2 minutes on 16 cores).

Each is the acceptance bar: cosine >= 0.9997 and max|err| <= 2e-2 max|ref|.
"""
import os
import sys

import numpy as np
import pytest

from diffusion_transformer_denoiser_amd import moss, synth
from oracle import dit_block as ob

from . import gates
from . import gpu_util as G

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
from make_stack_golden import input_digest, row_sketch, sketch_matrix  # noqa: E402


@pytest.fixture(scope="module")
def stack24():
    """(geometry, activation bits, [weight bits per block], GPU output as float64)."""
    t = G.torch()
    assert t.cuda.is_available(), "no GPU visible"
    assert moss.moss_device_check(0) == moss.MOSS_OK, "device 0 is not gfx950"
    geom = synth.CONFIGS["c4"]
    G.say(f"stack c4 x{geom.n_blocks}: generating inputs")
    acts = synth.make_activations(geom, 0)
    bits, dev_w = [], []
    for i in range(geom.n_blocks):
        wb = synth.make_block_weights(geom, 0, i)
        bits.append(wb)
        dev_w.append({k: G.dev(v) for k, v in wb.items()})
    dims = G.geometry_dims(geom)
    rope = G.empty_f32(2, geom.rows, 64)
    moss.moss_rope_build(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, rope)
    ws = t.empty(moss.moss_workspace_bytes(dims, geom.n_blocks), dtype=t.uint8, device="cuda")
    out = G.empty_bf16(geom.batch, geom.rows, geom.d_model)
    G.say("  stack forward")
    moss.moss_stack_forward(dims, dev_w, G.dev(acts["x"]), G.dev(acts["txt"]), acts["txt_len"], G.dev(acts["cond"]),
                            rope, out, ws)
    G.sync()
    got = G.host_f64(out)
    del dev_w, ws, out
    t.cuda.empty_cache()
    return geom, acts, bits, got


def _h0(acts):
    return ob.join_rows(ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), acts["txt_len"])


def test_stack24_against_the_record(stack24):
    """Sampled rows element by element, and every row of both items through its sketch."""
    geom, acts, bits, got = stack24
    gold = np.load(os.path.join(GOLDEN, "stack24_c4_rows.npz"))
    assert input_digest(acts, bits[0]) == str(gold["input_sha256"]), "seeded inputs differ from the record's"
    h0 = _h0(acts)
    rows = gold["rows"]
    ref = gold["values"].astype(np.float64)
    for b in range(geom.batch):
        G.assert_parity(f"item {b} sampled rows", got[b, rows], ref[b])
        G.assert_parity(f"item {b} sampled rows - h0", got[b, rows] - h0[b, rows], ref[b] - h0[b, rows])
    r = sketch_matrix(geom.d_model)
    n_out, p_out = row_sketch(got, r)
    n_upd, p_upd = row_sketch(got - h0, r)
    for b in range(geom.batch):
        G.assert_parity(f"item {b} row norms", n_out[b], gold["norm_out"][b])
        G.assert_parity(f"item {b} row projections", p_out[b], gold["proj_out"][b].astype(np.float64))
        G.assert_parity(f"item {b} update row norms", n_upd[b], gold["norm_upd"][b])
        G.assert_parity(f"item {b} update row projections", p_upd[b], gold["proj_upd"][b].astype(np.float64))
    G.say(f"  max|out| {np.max(np.abs(got), axis=(1, 2))} vs {gold['max_abs']}")
    assert np.allclose(np.max(np.abs(got), axis=(1, 2)), gold["max_abs"], rtol=2e-2)


def test_stack24_every_element(stack24):
    """The oracle's whole 24-block output, computed here on the host's cores, against every element."""
    geom, acts, bits, got = stack24
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)

    def blocks():
        for i, wb in enumerate(bits):
            G.say(f"  oracle block {i + 1}/{len(bits)}")
            yield ob.weights_f64(wb)

    ref = ob.stack_forward(ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), acts["txt_len"],
                           ob.widen_bf16(acts["cond"]), blocks(), cos, sin, geom.eps)
    h0 = _h0(acts)
    for b in range(geom.batch):
        G.say(f"item {b}, every element:")
        gates.check_block(got[b], ref[b], h0[b])
