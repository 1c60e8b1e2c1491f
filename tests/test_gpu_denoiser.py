"""One whole denoiser forward (the ends around the stack) against the float64
oracle (GPU): moss_denoiser_forward on seeded latents, prompt rows and
timesteps, gated by the acceptance bar (cosine >= 0.9997, max|err| <= 2e-2
max|ref|) on the velocity."""
import numpy as np
import pytest

from diffusion_transformer_denoiser_amd import moss, synth
from oracle import denoiser as od
from oracle import dit_block as ob

from . import gpu_util as G
from .test_gpu_block import STRONG

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    t = G.torch()
    assert t.cuda.is_available(), "no GPU visible"
    assert moss.moss_device_check(0) == moss.MOSS_OK, "device 0 is not gfx950"
    return t


def _case(geom, seed, enc_dim, n_blocks, std):
    inp = synth.make_denoiser_inputs(geom, seed, enc_dim)
    ends = synth.make_ends_weights(geom, seed, enc_dim, std)
    ws = [synth.make_block_weights(geom, seed, i, std=std) for i in range(n_blocks)]
    return inp, ends, ws


def _gpu(geom, inp, ends, ws, enc_dim, skip=None):
    t = G.torch()
    dims = G.geometry_dims(geom)
    rope = G.empty_f32(2, geom.rows, 64)
    moss.moss_rope_build(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, rope)
    workspace = t.empty(moss.moss_denoiser_workspace_bytes(dims, len(ws)), dtype=t.uint8, device="cuda")
    vel = G.empty_bf16(geom.batch, geom.n_img, 128)
    dev_ends = {k: G.dev(v) for k, v in ends.items()}
    dev_w = [{k: G.dev(v) for k, v in w.items()} for w in ws]
    moss.moss_denoiser_forward(dims, dev_w, G.dev(inp["latent"]), G.dev(inp["enc"]), inp["txt_len"], inp["t"],
                               dev_ends, enc_dim, rope, vel, workspace, skip=skip)
    G.sync()
    return vel


def _oracle(geom, inp, ends, ws, rounded=False, skip=None):
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    return od.denoiser_forward(ob.widen_bf16(inp["latent"]), ob.widen_bf16(inp["enc"]), inp["txt_len"],
                               inp["t"].astype(np.float64), {k: ob.widen_bf16(v) for k, v in ends.items()},
                               [ob.weights_f64(w) for w in ws], cos, sin, geom.eps, rounded=rounded, skip=skip)


@pytest.mark.parametrize("batch,lens,n_blocks", [(1, None, 1), (2, (8, 3), 2)])
def test_denoiser_small(batch, lens, n_blocks):
    kw = {"batch": batch}
    if lens is not None:
        kw["txt_len"] = lens
    geom = synth.smaller(synth.CONFIGS["c0"], **kw)
    G.say(f"denoiser c0-strong batch {batch} x{n_blocks}")
    inp, ends, ws = _case(geom, 11, 256, n_blocks, STRONG)
    got = G.host_f64(_gpu(geom, inp, ends, ws, 256))
    G.assert_parity("velocity", got, _oracle(geom, inp, ends, ws))
    G.assert_parity("velocity (rounding points)", got, _oracle(geom, inp, ends, ws, rounded=True))


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_denoiser_full_width(name):
    """D = 3072, encoder width 4096, one block: the released geometry's ends."""
    geom = synth.CONFIGS[name]
    G.say(f"denoiser {name}: {geom.n_txt}+{geom.n_img} rows, enc 4096")
    inp, ends, ws = _case(geom, 12, synth.ENC_DIM, 1, 0.02)
    got = G.host_f64(_gpu(geom, inp, ends, ws, synth.ENC_DIM))
    G.say("  oracle ...")
    G.assert_parity("velocity", got, _oracle(geom, inp, ends, ws))


def test_denoiser_skip_and_repeat():
    """A block skipped for one item of the guidance pair; two calls give the same bytes."""
    geom = synth.smaller(synth.CONFIGS["c0"], batch=2, txt_len=(8, 5))
    G.say("denoiser c0-strong x3 with a skipped block")
    inp, ends, ws = _case(geom, 13, 128, 3, STRONG)
    skip = [[False, False], [False, True], [False, False]]
    v1 = _gpu(geom, inp, ends, ws, 128, skip=skip).cpu().numpy()
    v2 = _gpu(geom, inp, ends, ws, 128, skip=skip).cpu().numpy()
    np.testing.assert_array_equal(v1, v2)
    got = ob.widen_bf16(v1.view(np.uint16))
    G.assert_parity("velocity", got, _oracle(geom, inp, ends, ws, skip=skip))
