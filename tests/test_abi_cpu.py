"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments before any HIP call (no GPU needed).

Pointers here are fake device addresses: validation never dereferences them.
"""
import ctypes

import pytest

from diffusion_transformer_denoiser_amd import moss

BASE = 1 << 40
MB = 1_000_000


def fake(i, offset=0):
    """A distinct, 16-byte aligned fake device address per slot i."""
    return BASE + i * (1 << 34) + offset


def c2_dims(**kw):
    d = dict(batch=1, n_img=4096, n_txt=34, d_model=3072, mlp_inner=12288, eps=1e-6)
    d.update(kw)
    return moss.make_dims(**d)


def weights(base_slot=10):
    return moss.moss_block_weights(*[fake(base_slot + i) for i in range(7)])


def block(dims, ws_bytes=None, txt_len=None, x=None, txt=None, out=None, ws=None, cond=None, rope=None, w=None):
    L = moss.lib()
    if ws_bytes is None:
        ws_bytes = moss.moss_workspace_bytes(dims, 1)
    lens = None
    if txt_len is not None:
        lens = ctypes.cast((ctypes.c_int32 * len(txt_len))(*txt_len), ctypes.c_void_p)
    return L.moss_block_forward(ctypes.byref(dims), fake(1) if x is None else x, fake(2) if txt is None else txt,
                                lens, fake(3) if cond is None else cond, ctypes.byref(w or weights()),
                                fake(4) if rope is None else rope, fake(5) if out is None else out,
                                fake(6) if ws is None else ws, ws_bytes, None)


def test_library_exports_every_declared_function():
    L = moss.lib()
    names = moss.declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n


def test_binding_covers_every_declared_function():
    for n in moss.declared_functions():
        assert callable(getattr(moss, n, None)), n


def test_status_strings():
    for s in range(6):
        assert moss.moss_status_string(s)
    assert moss.moss_status_string(99) == "unknown status"


def test_workspace_bytes():
    d = c2_dims()
    ws = moss.moss_workspace_bytes(d, 1)
    # fp32 residual (50.7 MB) + a (25.4 MB) + packed q/k/v (3 x 26.0 MB) + z (101.5 MB)
    assert 250 * MB < ws < 260 * MB, ws
    # every block's modulation [B, 6D] fp32 is computed up front: 73.7 KB more per block at B = 1
    assert moss.moss_workspace_bytes(d, 24) - ws == 23 * 4 * 6 * 3072
    assert moss.moss_workspace_bytes(c2_dims(batch=2), 1) > ws
    assert moss.moss_workspace_bytes(c2_dims(head_dim=64), 1) == 0
    assert moss.moss_workspace_bytes(d, 0) == 0


def test_packed_rows():
    assert moss.moss_packed_rows(4130) == 4224
    assert moss.moss_packed_rows(128) == 128
    assert moss.moss_packed_rows(1) == 128
    assert moss.moss_packed_rows(0) == 0


@pytest.mark.parametrize("kw", [
    dict(head_dim=64), dict(d_model=3000), dict(n_heads=23), dict(mlp_inner=12280), dict(mlp_inner=0),
    dict(eps=0.0), dict(eps=-1.0), dict(eps=float("inf")), dict(batch=0), dict(batch=17), dict(n_img=-1),
    dict(n_img=0, n_txt=0), dict(n_img=70000), dict(d_model=16384, n_heads=128),
])
def test_block_rejects_bad_dims(kw):
    assert block(c2_dims(**kw)) == moss.MOSS_EINVAL


@pytest.mark.parametrize("lens", [[35], [-1], [34, 35]])
def test_block_rejects_bad_txt_len(lens):
    d = c2_dims(batch=len(lens))
    assert block(d, txt_len=lens) == moss.MOSS_EINVAL


def test_block_rejects_no_valid_row():
    d = c2_dims(n_img=0, n_txt=8)
    assert block(d, txt_len=[0]) == moss.MOSS_EINVAL


@pytest.mark.parametrize("which", ["x", "txt", "cond", "rope", "out"])
def test_block_rejects_null_and_misaligned(which):
    assert block(c2_dims(), **{which: 0}) == moss.MOSS_EINVAL
    assert block(c2_dims(), **{which: fake(1 + ["x", "txt", "cond", "rope", "out"].index(which), 8)}) == moss.MOSS_EINVAL


def test_block_rejects_bad_weights():
    w = weights()
    w.w_up = None
    assert block(c2_dims(), w=w) == moss.MOSS_EINVAL
    w = weights()
    w.q_gain = fake(13, 2)
    assert block(c2_dims(), w=w) == moss.MOSS_EINVAL


def test_block_workspace_errors():
    d = c2_dims()
    need = moss.moss_workspace_bytes(d, 1)
    assert block(d, ws_bytes=need - 1) == moss.MOSS_EWORKSPACE
    assert block(d, ws=0) == moss.MOSS_EWORKSPACE


def test_block_rejects_aliasing():
    d = c2_dims()
    assert block(d, out=fake(6, 1 << 20)) == moss.MOSS_EALIAS  # out inside the workspace
    assert block(d, out=fake(1, 4096)) == moss.MOSS_EALIAS  # out overlaps x
    assert block(d, out=fake(14, 1 << 20)) == moss.MOSS_EALIAS  # out overlaps w_out


@pytest.mark.parametrize("which", ["x", "txt", "cond", "rope"])
def test_block_rejects_input_in_workspace(which):
    """An input that lies in the workspace would be overwritten during the call."""
    assert block(c2_dims(), **{which: fake(6, 1 << 20)}) == moss.MOSS_EALIAS


def test_block_rejects_weights_in_workspace():
    w = weights()
    w.w_down = fake(6, 4 << 20)
    assert block(c2_dims(), w=w) == moss.MOSS_EALIAS
    L = moss.lib()
    ws = (moss.moss_block_weights * 2)(weights(), weights(20))
    ws[1].q_gain = fake(6, 256)
    d = c2_dims()
    assert L.moss_stack_forward(ctypes.byref(d), 2, fake(1), fake(2), None, fake(3), ws, fake(4), fake(5), fake(6),
                                moss.moss_workspace_bytes(d, 2), None) == moss.MOSS_EALIAS


def test_valid_call_without_gpu_reports_device():
    """With valid arguments the call reaches the device check; here there is no GPU."""
    if moss.moss_device_check(0) == moss.MOSS_OK:
        pytest.skip("a gfx950 device is present")
    assert block(c2_dims()) == moss.MOSS_EDEVICE
    assert moss.lib().moss_rope_build(34, 64, 64, 10000.0, fake(4), None) == moss.MOSS_EDEVICE


def test_stack_rejects_zero_blocks():
    L = moss.lib()
    d = c2_dims()
    rc = L.moss_stack_forward(ctypes.byref(d), 0, fake(1), fake(2), None, fake(3), ctypes.byref(weights()), fake(4),
                              fake(5), fake(6), moss.moss_workspace_bytes(d, 1), None)
    assert rc == moss.MOSS_EINVAL


def test_single_step_entry_points_validate():
    L = moss.lib()
    assert L.moss_k_gemm_nt(100, 200, 256, fake(1), 256, fake(2), 256, fake(3), 200, None) == moss.MOSS_EINVAL
    assert L.moss_k_gemm_nt(100, 256, 192, fake(1), 192, fake(2), 192, fake(3), 256, None) == moss.MOSS_EINVAL
    assert L.moss_k_gemm_nt(100, 256, 64, fake(1), 64, fake(2), 64, fake(3), 256, None) == moss.MOSS_EINVAL
    assert L.moss_k_gemm_nt(100, 256, 256, fake(1), 100, fake(2), 256, fake(3), 256, None) == moss.MOSS_EINVAL
    assert L.moss_k_gemm_nt(100, 256, 256, fake(1), 256, fake(2), 256, fake(1, 512), 256, None) == moss.MOSS_EALIAS
    assert L.moss_k_silu_mul(10, 100, fake(1), fake(2), None) == moss.MOSS_EINVAL
    assert L.moss_k_silu_mul(10, 128, fake(1), fake(1, 64), None) == moss.MOSS_EALIAS
    assert L.moss_k_gated_add(1, 10, 256, fake(1), fake(2), 100, fake(3), None, None) == moss.MOSS_EINVAL
    assert L.moss_k_gated_add(1, 10, 256, fake(1), fake(2), 1536, fake(3), fake(1, 64), None) == moss.MOSS_EALIAS
    assert L.moss_k_mod_rmsnorm(1, 10, 256, 0.0, fake(1), fake(2), fake(3), 1536, fake(4), None) == moss.MOSS_EINVAL
    assert L.moss_k_attention(1, 2, 10, 11, None, fake(1), fake(2), fake(3), fake(4), None) == moss.MOSS_EINVAL
    assert L.moss_k_qk_norm_rope_pack(1, 10, 2, 1e-6, fake(1), fake(2), fake(3), fake(4), fake(5), fake(5), fake(6),
                                      None) == moss.MOSS_EALIAS
    assert L.moss_k_adaln_gemv(1, 256, fake(1), fake(2), fake(3), fake(4), 100, None) == moss.MOSS_EWORKSPACE
    # the fused QKV step: 10 rows pack to 128, so it needs 512 * 128 bytes of workspace
    qkv_args = (1, 10, 2, 1e-6, fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(8))
    assert L.moss_k_gemm_qkv_pack(*qkv_args, fake(9), 512 * 128 - 1, None) == moss.MOSS_EWORKSPACE
    assert L.moss_k_gemm_qkv_pack(*qkv_args, None, 512 * 128, None) == moss.MOSS_EWORKSPACE
    assert L.moss_k_gemm_qkv_pack(*qkv_args, fake(6), 512 * 128, None) == moss.MOSS_EALIAS  # workspace on q
    assert L.moss_k_gemm_qkv_pack(1, 10, 2, 0.0, *qkv_args[4:], fake(9), 512 * 128, None) == moss.MOSS_EINVAL
    assert L.moss_rope_build(-1, 4, 4, 10000.0, fake(1), None) == moss.MOSS_EINVAL
    assert L.moss_rope_build(2, 4, 4, 1.0, fake(1), None) == moss.MOSS_EINVAL


def test_fused_gemm_entry_points_validate():
    L = moss.lib()
    assert L.moss_k_gemm_silu(100, 200, 256, fake(1), 256, fake(2), 256, fake(3), 200, None) == moss.MOSS_EINVAL
    assert L.moss_k_gemm_silu(100, 256, 256, fake(1), 256, fake(2), 256, fake(2, 4096), 256, None) == moss.MOSS_EALIAS
    assert L.moss_k_gemm_gated_add(100, 256, 256, fake(1), 256, fake(2), 256, fake(3), fake(4), 1536, 30, None,
                                   None) == moss.MOSS_EINVAL  # 100 rows are not whole items of 30
    assert L.moss_k_gemm_gated_add(100, 256, 256, fake(1), 256, fake(2), 256, fake(3), fake(4), 100, 100, None,
                                   None) == moss.MOSS_EINVAL  # gate stride below n
    assert L.moss_k_gemm_gated_add(100, 256, 256, fake(1), 256, fake(2), 256, fake(3), fake(4), 1536, 100,
                                   fake(3, 256), None) == moss.MOSS_EALIAS  # out inside h


def test_probe_arguments():
    L = moss.lib()
    assert L.moss_probe_arm(-1, 4, 1) == moss.MOSS_EINVAL
    assert L.moss_probe_arm(13, 4, 1) == moss.MOSS_EINVAL
    assert L.moss_probe_arm(3, 0, 1) == moss.MOSS_EINVAL
    assert L.moss_probe_arm(3, 4, 0) == moss.MOSS_EINVAL
    assert L.moss_probe_collect(None, -1) == -moss.MOSS_EINVAL


def test_guidance_euler_validates():
    L = moss.lib()
    ok = (fake(1), fake(2), 3.0, -0.02, fake(3), fake(4), None)
    assert L.moss_guidance_euler(10, 12, *ok) == moss.MOSS_EINVAL  # width % 8
    assert L.moss_guidance_euler(-1, 16, *ok) == moss.MOSS_EINVAL
    assert L.moss_guidance_euler(10, 16, fake(1), None, 3.0, -0.02, fake(3), fake(4), None) == moss.MOSS_EINVAL
    assert L.moss_guidance_euler(10, 16, fake(1), fake(2), float("nan"), -0.02, fake(3), fake(4), None) == \
        moss.MOSS_EINVAL
    assert L.moss_guidance_euler(10, 16, fake(1), fake(2), 3.0, float("inf"), fake(3), fake(4), None) == \
        moss.MOSS_EINVAL
    assert L.moss_guidance_euler(10, 16, fake(1, 8), fake(2), 3.0, -0.02, fake(3), fake(4), None) == moss.MOSS_EINVAL
    assert L.moss_guidance_euler(10, 16, fake(1), fake(2), 3.0, -0.02, fake(3), fake(1, 64), None) == \
        moss.MOSS_EALIAS  # x_out over v_pos
    assert L.moss_guidance_euler(10, 16, fake(1), fake(2), 3.0, -0.02, fake(3), fake(3, 32), None) == \
        moss.MOSS_EALIAS  # x_out partly over x_in
    assert L.moss_guidance_euler(0, 16, *ok) == moss.MOSS_OK  # nothing to do, no device needed
    if moss.moss_device_check(0) != moss.MOSS_OK:
        assert L.moss_guidance_euler(10, 16, *ok) == moss.MOSS_EDEVICE
        assert L.moss_guidance_euler(10, 16, fake(1), None, 1.0, -0.02, fake(3), fake(3), None) == \
            moss.MOSS_EDEVICE  # guidance 1 without the negative pass, in place


def test_stack_skip_validates():
    L = moss.lib()
    d = c2_dims()
    flags = (ctypes.c_uint8 * 2)(0, 1)
    rc = L.moss_stack_forward_skip(ctypes.byref(d), 0, fake(1), fake(2), None, fake(3), ctypes.byref(weights()),
                                   ctypes.cast(flags, ctypes.c_void_p), fake(4), fake(5), fake(6),
                                   moss.moss_workspace_bytes(d, 1), None)
    assert rc == moss.MOSS_EINVAL
    if moss.moss_device_check(0) != moss.MOSS_OK:
        rc = L.moss_stack_forward_skip(ctypes.byref(d), 1, fake(1), fake(2), None, fake(3), ctypes.byref(weights()),
                                       ctypes.cast(flags, ctypes.c_void_p), fake(4), fake(5), fake(6),
                                       moss.moss_workspace_bytes(d, 1), None)
        assert rc == moss.MOSS_EDEVICE


def _ends(enc_dim=4096, base_slot=30):
    return moss.moss_denoiser_weights(*[fake(base_slot + i) for i in range(6)], enc_dim)


def denoiser(dims, n_blocks=1, ends=None, latent=None, enc=None, t=(500.0,), vel=None, ws=None, ws_bytes=None,
             lens=None):
    L = moss.lib()
    if ws_bytes is None:
        ws_bytes = moss.moss_denoiser_workspace_bytes(dims, n_blocks)
    ts = (ctypes.c_float * len(t))(*t)
    blocks = (moss.moss_block_weights * n_blocks)(*[weights() for _ in range(n_blocks)])
    ln = None if lens is None else ctypes.cast((ctypes.c_int32 * len(lens))(*lens), ctypes.c_void_p)
    return L.moss_denoiser_forward(ctypes.byref(dims), n_blocks, fake(1) if latent is None else latent,
                                   fake(2) if enc is None else enc, ln, ctypes.cast(ts, ctypes.c_void_p),
                                   ctypes.byref(ends or _ends()), blocks, None, fake(4), fake(5) if vel is None else vel,
                                   fake(6) if ws is None else ws, ws_bytes, None)


def test_denoiser_workspace_bytes():
    d = c2_dims()
    assert moss.moss_denoiser_workspace_bytes(d, 1) > moss.moss_workspace_bytes(d, 1)
    assert moss.moss_denoiser_workspace_bytes(c2_dims(n_img=0, n_txt=8), 1) == 0
    assert moss.moss_denoiser_workspace_bytes(d, 0) == 0


def test_denoiser_validates():
    d = c2_dims()
    assert denoiser(d, ends=_ends(enc_dim=100)) == moss.MOSS_EINVAL
    assert denoiser(d, ends=_ends(enc_dim=0)) == moss.MOSS_EINVAL
    assert denoiser(d, t=(float("nan"),)) == moss.MOSS_EINVAL
    assert denoiser(d, latent=0) == moss.MOSS_EINVAL
    assert denoiser(d, latent=fake(1, 8)) == moss.MOSS_EINVAL
    assert denoiser(d, n_blocks=0) == moss.MOSS_EINVAL
    assert denoiser(c2_dims(n_img=0, n_txt=8), lens=[8]) == moss.MOSS_EINVAL
    e = _ends()
    e.w_final = None
    assert denoiser(d, ends=e) == moss.MOSS_EINVAL
    need = moss.moss_denoiser_workspace_bytes(d, 1)
    assert denoiser(d, ws_bytes=need - 1) == moss.MOSS_EWORKSPACE
    assert denoiser(d, vel=fake(6, 4096)) == moss.MOSS_EALIAS  # velocity inside the workspace
    assert denoiser(d, vel=fake(1, 256)) == moss.MOSS_EALIAS  # velocity over the latent
    assert denoiser(d, vel=fake(35, 0)) == moss.MOSS_EALIAS  # velocity over w_final
    assert denoiser(d, latent=fake(6, 4096)) == moss.MOSS_EALIAS  # latent inside the workspace
    e = _ends()
    e.w_t2 = fake(6, 1 << 20)
    assert denoiser(d, ends=e) == moss.MOSS_EALIAS  # a weight of the ends inside the workspace
    if moss.moss_device_check(0) != moss.MOSS_OK:
        assert denoiser(d) == moss.MOSS_EDEVICE


def test_noalloc_block_validates():
    """The no-allocation block forward: a geometry whose workspace exceeds the library's scratch is
    refused before any HIP call; a fitting one reaches the device check (no GPU here)."""
    L = moss.lib()
    assert moss.moss_noalloc_scratch_bytes() == 256 << 20
    big = c2_dims(batch=2)
    assert moss.moss_workspace_bytes(big, 1) > moss.moss_noalloc_scratch_bytes()
    args = (fake(1), fake(2), None, fake(3), ctypes.byref(weights()), fake(4), fake(5), None)
    assert L.moss_block_forward_noalloc(ctypes.byref(big), *args) == moss.MOSS_EWORKSPACE
    bad = c2_dims(d_model=3000)
    assert L.moss_block_forward_noalloc(ctypes.byref(bad), *args) == moss.MOSS_EINVAL
    if moss.moss_device_check(0) != moss.MOSS_OK:
        assert L.moss_block_forward_noalloc(ctypes.byref(c2_dims()), *args) == moss.MOSS_EDEVICE
