"""The block forward captured in a HIP graph (GPU).

The library launches only kernels (no allocation, no memset, no host
synchronisation), so a caller may capture a whole block into a graph and
replay it.  Each replay must reproduce the eager output bit for bit, with the
program's own eager work and synchronisations between replays."""
import numpy as np
import pytest

from diffusion_transformer_denoiser_amd import moss, synth

from . import gpu_util as G
from .test_gpu_block import STRONG

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,batch,lens", [("c0", 2, (8, 3)), ("c1", 1, None)])
def test_block_graph_replays_match_eager(name, batch, lens):
    t = G.torch()
    assert moss.moss_device_check(0) == moss.MOSS_OK
    kw = {"batch": batch}
    if lens is not None:
        kw["txt_len"] = lens
    geom = synth.smaller(synth.CONFIGS[name], **kw)
    G.say(f"graph capture of the {name} block, batch {batch}")
    acts = synth.make_activations(geom, 9)
    w = synth.make_block_weights(geom, 9, 0, std=STRONG if name == "c0" else 0.02)
    dims = G.geometry_dims(geom)
    rope = G.empty_f32(2, geom.rows, 64)
    moss.moss_rope_build(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, rope)
    ws = t.empty(moss.moss_workspace_bytes(dims, 1), dtype=t.uint8, device="cuda")
    out = G.empty_bf16(geom.batch, geom.rows, geom.d_model)
    w_dev = {k: G.dev(v) for k, v in w.items()}  # the tensors must outlive every call and replay
    dev_w = moss.make_weights(w_dev)
    x, txt, cond = G.dev(acts["x"]), G.dev(acts["txt"]), G.dev(acts["cond"])

    def step():
        moss.moss_block_forward(dims, x, txt, acts["txt_len"], cond, dev_w, rope, out, ws)

    step()
    G.sync()
    eager = out.cpu().numpy().copy()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):  # warm-up on the capture stream's kind of stream, as torch recommends
        step()
    t.cuda.current_stream().wait_stream(side)
    G.sync()
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        step()
    G.sync()
    scratch = t.ones(1 << 20, device="cuda")
    for r in range(4):
        out.fill_(0)
        scratch.mul_(1.5)  # the program's own eager work between replays
        graph.replay()
        G.sync()
        np.testing.assert_array_equal(out.cpu().numpy(), eager, err_msg=f"replay {r}")
        step()  # an eager call between replays leaves the graph's result unchanged
        G.sync()
        np.testing.assert_array_equal(out.cpu().numpy(), eager, err_msg=f"eager after replay {r}")
