"""The no-allocation block forward against moss_block_forward (GPU).

moss_block_forward_noalloc runs the same kernels with the library's own scratch
array instead of a workspace argument: two calls in a row (the 4096+34-row
block, then a smaller two-item geometry) must each give the bytes
moss_block_forward gives on the same inputs, and a geometry whose workspace
exceeds the scratch is refused.
"""
import ctypes

import numpy as np
import pytest

from diffusion_transformer_denoiser_amd import moss, synth
from oracle import dit_block as ob

from . import gates
from . import gpu_util as G

pytestmark = pytest.mark.gpu


def _inputs(geom, seed, std):
    acts = synth.make_activations(geom, seed)
    w = synth.make_block_weights(geom, seed, 0, std=std)
    dims = G.geometry_dims(geom)
    rope = G.empty_f32(2, geom.rows, 64)
    moss.moss_rope_build(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, rope)
    dev = dict(x=G.dev(acts["x"]), txt=G.dev(acts["txt"]), cond=G.dev(acts["cond"]),
               w={k: G.dev(v) for k, v in w.items()})
    return acts, w, dims, rope, dev


def test_noalloc_matches_block_forward_twice():
    t = G.torch()
    assert t.cuda.is_available(), "no GPU visible"
    assert moss.moss_device_check(0) == moss.MOSS_OK, "device 0 is not gfx950"
    assert moss.moss_noalloc_scratch_bytes() == 256 << 20
    cases = [(synth.CONFIGS["c2"], 0, 0.02),
             (synth.smaller(synth.CONFIGS["c0"], batch=2, txt_len=(8, 3)), 14, 0.02 * np.sqrt(3072 / 256))]
    for geom, seed, std in cases:
        G.say(f"noalloc block {geom.name}: B={geom.batch} rows={geom.rows} D={geom.d_model}")
        acts, w, dims, rope, dev = _inputs(geom, seed, std)
        assert moss.moss_workspace_bytes(dims, 1) <= moss.moss_noalloc_scratch_bytes()
        ws = t.empty(moss.moss_workspace_bytes(dims, 1), dtype=t.uint8, device="cuda")
        ref_out = G.empty_bf16(geom.batch, geom.rows, geom.d_model)
        moss.moss_block_forward(dims, dev["x"], dev["txt"], acts["txt_len"], dev["cond"], dev["w"], rope, ref_out, ws)
        out = G.empty_bf16(geom.batch, geom.rows, geom.d_model)
        out.fill_(0x7FC0)
        moss.moss_block_forward_noalloc(dims, dev["x"], dev["txt"], acts["txt_len"], dev["cond"], dev["w"], rope, out)
        G.sync()
        got, ref = G.host_bits(out), G.host_bits(ref_out)
        G.say(f"  {np.mean(got == ref) * 100:.4f}% of the output bytes equal")
        np.testing.assert_array_equal(got, ref)
        if geom.d_model == 256:  # the small call against the oracle too
            cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
            x, txt, cond = ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), ob.widen_bf16(acts["cond"])
            oref = ob.block_forward(x, txt, acts["txt_len"], cond, ob.weights_f64(w), cos, sin, geom.eps)
            gates.check_block(ob.widen_bf16(got), oref, ob.join_rows(x, txt, acts["txt_len"]))
        del ws


def test_noalloc_refuses_a_geometry_beyond_the_scratch():
    """Two items of 4130 rows need 490 MiB of workspace: MOSS_EWORKSPACE, before any launch."""
    d = moss.make_dims(2, 4096, 34, 3072, 12288, 1e-6)
    w = moss.moss_block_weights(*[16 * (i + 1) << 30 for i in range(7)])
    rc = moss.lib().moss_block_forward_noalloc(ctypes.byref(d), 1 << 40, 2 << 40, None, 3 << 40, ctypes.byref(w),
                                               4 << 40, 5 << 40, None)
    assert rc == moss.MOSS_EWORKSPACE
