"""Thin ctypes binding of libmoss.so (the C ABI in include/moss.h).

Argument marshalling only: every function here has the name of the C entry
point it calls, turns torch tensors into device pointers and a torch stream
into a hipStream_t, and raises ``MossError`` on a non-zero status.  All
compute runs in the HIP kernels of the library.  If the library is not built
the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoss.so")
# A differently built copy of the library (the host-sanitizer build the CPU tests run against) may be
# named here; the product path loads libmoss.so.
LIB_PATH = os.environ.get("MOSS_LIBRARY", LIB_PATH)
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moss.h")

MOSS_OK, MOSS_EINVAL, MOSS_EALIAS, MOSS_EWORKSPACE, MOSS_EDEVICE, MOSS_EHIP = range(6)
HEAD_DIM = 128
STEPS = ("JOIN", "ADALN", "NORM1", "QKV", "QKNORM", "ATTN", "OUT", "GATE1", "NORM2", "UP", "SILU", "DOWN", "GATE2")
STEP = {name: i for i, name in enumerate(STEPS)}

c_i32, c_f32, c_vp, c_size = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class moss_dims(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("n_img", c_i32), ("n_txt", c_i32), ("d_model", c_i32), ("n_heads", c_i32),
                ("head_dim", c_i32), ("mlp_inner", c_i32), ("eps", c_f32)]


WEIGHT_FIELDS = ("w_mod", "w_qkv", "q_gain", "k_gain", "w_out", "w_up", "w_down")


class moss_block_weights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in WEIGHT_FIELDS]


END_FIELDS = ("w_t1", "w_t2", "w_txt", "w_in", "w_fmod", "w_final")


class moss_denoiser_weights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in END_FIELDS] + [("enc_dim", ctypes.c_int32)]


class MossError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moss_status_string(status)} (status {status})")


_SIGS = {
    "moss_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moss_device_check": (ctypes.c_int, [ctypes.c_int]),
    "moss_workspace_bytes": (c_size, [ctypes.POINTER(moss_dims), c_i32]),
    "moss_packed_rows": (c_i32, [c_i32]),
    "moss_rope_build": (ctypes.c_int, [c_i32, c_i32, c_i32, c_f32, c_vp, c_vp]),
    "moss_block_forward": (ctypes.c_int, [ctypes.POINTER(moss_dims), c_vp, c_vp, c_vp, c_vp,
                                          ctypes.POINTER(moss_block_weights), c_vp, c_vp, c_vp, c_size, c_vp]),
    "moss_block_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(moss_dims), c_vp, c_vp, c_vp, c_vp,
                                                  ctypes.POINTER(moss_block_weights), c_vp, c_vp, c_vp]),
    "moss_noalloc_scratch_bytes": (c_size, []),
    "moss_stack_forward": (ctypes.c_int, [ctypes.POINTER(moss_dims), c_i32, c_vp, c_vp, c_vp, c_vp,
                                          ctypes.POINTER(moss_block_weights), c_vp, c_vp, c_vp, c_size, c_vp]),
    "moss_stack_forward_skip": (ctypes.c_int, [ctypes.POINTER(moss_dims), c_i32, c_vp, c_vp, c_vp, c_vp,
                                               ctypes.POINTER(moss_block_weights), c_vp, c_vp, c_vp, c_vp, c_size,
                                               c_vp]),
    "moss_denoiser_workspace_bytes": (c_size, [ctypes.POINTER(moss_dims), c_i32]),
    "moss_denoiser_forward": (ctypes.c_int, [ctypes.POINTER(moss_dims), c_i32, c_vp, c_vp, c_vp, c_vp,
                                             ctypes.POINTER(moss_denoiser_weights), ctypes.POINTER(moss_block_weights),
                                             c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "moss_guidance_euler": (ctypes.c_int, [c_i32, c_i32, c_vp, c_vp, c_f32, c_f32, c_vp, c_vp, c_vp]),
    "moss_k_join_rows": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moss_k_adaln_gemv": (ctypes.c_int, [c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "moss_k_mod_rmsnorm": (ctypes.c_int, [c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp]),
    "moss_k_gemm_nt": (ctypes.c_int, [c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_vp, c_i32, c_vp]),
    "moss_k_qk_norm_rope_pack": (ctypes.c_int, [c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                c_vp, c_vp]),
    "moss_k_gemm_qkv_pack": (ctypes.c_int, [c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                            c_vp, c_vp, c_size, c_vp]),
    "moss_k_attention": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moss_k_silu_mul": (ctypes.c_int, [c_i32, c_i32, c_vp, c_vp, c_vp]),
    "moss_k_gated_add": (ctypes.c_int, [c_i32, c_i32, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "moss_k_gemm_silu": (ctypes.c_int, [c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_vp, c_i32, c_vp]),
    "moss_k_gemm_gated_add": (ctypes.c_int, [c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32,
                                             c_vp, c_vp]),
    "moss_probe_arm": (ctypes.c_int, [c_i32, c_i32, c_i32]),
    "moss_probe_collect": (c_i32, [ctypes.POINTER(ctypes.c_float), c_i32]),
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m diffusion_transformer_denoiser_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name, None)
            if fn is None:  # an older build: calling this entry point raises AttributeError
                continue
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def declared_functions() -> list:
    """Names of the functions include/moss.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moss_[a-z0-9_]+)\s*\(", text)))


# ---- marshalling --------------------------------------------------------------


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _lens(txt_len):
    if txt_len is None:
        return None
    arr = (c_i32 * len(txt_len))(*[int(n) for n in txt_len])
    return arr


def _check(rc: int, where: str) -> None:
    if rc != MOSS_OK:
        raise MossError(rc, where)


def make_dims(batch, n_img, n_txt, d_model, mlp_inner, eps=1e-6, n_heads=None, head_dim=HEAD_DIM) -> moss_dims:
    if n_heads is None:
        n_heads = d_model // head_dim
    return moss_dims(batch, n_img, n_txt, d_model, n_heads, head_dim, mlp_inner, eps)


def make_weights(w: dict) -> moss_block_weights:
    """The weight struct of one block; it keeps the tensors alive as long as it lives
    (the struct holds raw device pointers)."""
    s = moss_block_weights(*[_p(w[n]) for n in WEIGHT_FIELDS])
    s._tensors = [w[n] for n in WEIGHT_FIELDS]
    return s


# ---- the entry points -------------------------------------------------------------


def moss_status_string(status: int) -> str:
    return lib().moss_status_string(status).decode()


def moss_device_check(device: int = 0) -> int:
    return lib().moss_device_check(device)


def moss_workspace_bytes(dims: moss_dims, n_blocks: int = 1) -> int:
    return lib().moss_workspace_bytes(ctypes.byref(dims), n_blocks)


def moss_packed_rows(rows: int) -> int:
    return lib().moss_packed_rows(rows)


def moss_rope_build(n_txt, grid_h, grid_w, theta, rope, stream=None) -> None:
    _check(lib().moss_rope_build(n_txt, grid_h, grid_w, theta, _p(rope), _s(stream)), "moss_rope_build")


def moss_block_forward(dims, x, txt, txt_len, cond, weights, rope, out, workspace, stream=None) -> None:
    w = weights if isinstance(weights, moss_block_weights) else make_weights(weights)
    rc = lib().moss_block_forward(ctypes.byref(dims), _p(x), _p(txt), ctypes.cast(_lens(txt_len), c_vp), _p(cond),
                                  ctypes.byref(w), _p(rope), _p(out), _p(workspace),
                                  workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                  _s(stream))
    _check(rc, "moss_block_forward")


def moss_block_forward_noalloc(dims, x, txt, txt_len, cond, weights, rope, out, stream=None) -> None:
    w = weights if isinstance(weights, moss_block_weights) else make_weights(weights)
    rc = lib().moss_block_forward_noalloc(ctypes.byref(dims), _p(x), _p(txt), ctypes.cast(_lens(txt_len), c_vp),
                                          _p(cond), ctypes.byref(w), _p(rope), _p(out), _s(stream))
    _check(rc, "moss_block_forward_noalloc")


def moss_noalloc_scratch_bytes() -> int:
    return int(lib().moss_noalloc_scratch_bytes())


def moss_stack_forward(dims, blocks, x, txt, txt_len, cond, rope, out, workspace, stream=None) -> None:
    arr = (moss_block_weights * len(blocks))(
        *[b if isinstance(b, moss_block_weights) else make_weights(b) for b in blocks])
    rc = lib().moss_stack_forward(ctypes.byref(dims), len(blocks), _p(x), _p(txt),
                                  ctypes.cast(_lens(txt_len), c_vp), _p(cond), arr, _p(rope), _p(out),
                                  _p(workspace),
                                  workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                  _s(stream))
    _check(rc, "moss_stack_forward")


def moss_stack_forward_skip(dims, blocks, skip, x, txt, txt_len, cond, rope, out, workspace, stream=None) -> None:
    """``skip``: None, or n_blocks rows of batch flags (true = block not applied to that item)."""
    arr = (moss_block_weights * len(blocks))(
        *[b if isinstance(b, moss_block_weights) else make_weights(b) for b in blocks])
    sk = None
    if skip is not None:
        flat = [1 if f else 0 for row in skip for f in row]
        flags = (ctypes.c_uint8 * len(flat))(*flat)  # alive until the call returns
        sk = ctypes.cast(flags, c_vp)
    rc = lib().moss_stack_forward_skip(ctypes.byref(dims), len(blocks), _p(x), _p(txt),
                                       ctypes.cast(_lens(txt_len), c_vp), _p(cond), arr, sk, _p(rope), _p(out),
                                       _p(workspace),
                                       workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                       _s(stream))
    _check(rc, "moss_stack_forward_skip")


def make_ends(e: dict, enc_dim: int) -> moss_denoiser_weights:
    """The ends' weight struct; it keeps the tensors alive as long as it lives."""
    s = moss_denoiser_weights(*[_p(e[n]) for n in END_FIELDS], enc_dim)
    s._tensors = [e[n] for n in END_FIELDS]
    return s


def moss_denoiser_workspace_bytes(dims, n_blocks) -> int:
    return lib().moss_denoiser_workspace_bytes(ctypes.byref(dims), n_blocks)


def moss_denoiser_forward(dims, blocks, latent, enc, txt_len, t, ends, enc_dim, rope, velocity, workspace,
                          skip=None, stream=None) -> None:
    """``ends``: a dict of the six end weights (or a moss_denoiser_weights); ``t``: per-item timesteps."""
    arr = (moss_block_weights * len(blocks))(
        *[b if isinstance(b, moss_block_weights) else make_weights(b) for b in blocks])
    e = ends if isinstance(ends, moss_denoiser_weights) else make_ends(ends, enc_dim)
    ts = (ctypes.c_float * len(t))(*[float(v) for v in t])
    sk = None
    if skip is not None:
        flat = [1 if f else 0 for row in skip for f in row]
        flags = (ctypes.c_uint8 * len(flat))(*flat)  # alive until the call returns
        sk = ctypes.cast(flags, c_vp)
    rc = lib().moss_denoiser_forward(ctypes.byref(dims), len(blocks), _p(latent), _p(enc),
                                     ctypes.cast(_lens(txt_len), c_vp), ctypes.cast(ts, c_vp), ctypes.byref(e), arr, sk,
                                     _p(rope), _p(velocity), _p(workspace),
                                     workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                     _s(stream))
    _check(rc, "moss_denoiser_forward")


def moss_guidance_euler(rows, width, v_pos, v_neg, guidance, dsigma, x_in, x_out, stream=None) -> None:
    _check(lib().moss_guidance_euler(rows, width, _p(v_pos), _p(v_neg), guidance, dsigma, _p(x_in), _p(x_out),
                                     _s(stream)), "moss_guidance_euler")


def moss_k_join_rows(batch, n_txt, n_img, d_model, x, txt, txt_len, out, stream=None) -> None:
    _check(lib().moss_k_join_rows(batch, n_txt, n_img, d_model, _p(x), _p(txt), ctypes.cast(_lens(txt_len), c_vp),
                                  _p(out), _s(stream)), "moss_k_join_rows")


def moss_k_adaln_gemv(batch, d_model, cond, w_mod, mod, workspace, stream=None) -> None:
    _check(lib().moss_k_adaln_gemv(batch, d_model, _p(cond), _p(w_mod), _p(mod), _p(workspace),
                                   workspace.numel() * workspace.element_size(), _s(stream)), "moss_k_adaln_gemv")


def moss_k_mod_rmsnorm(batch, rows, d_model, eps, h, shift, scale, mod_stride, out, stream=None) -> None:
    _check(lib().moss_k_mod_rmsnorm(batch, rows, d_model, eps, _p(h), _p(shift), _p(scale), mod_stride, _p(out),
                                    _s(stream)), "moss_k_mod_rmsnorm")


def moss_k_gemm_nt(m, n, k, a, lda, w, ldw, c, ldc, stream=None) -> None:
    _check(lib().moss_k_gemm_nt(m, n, k, _p(a), lda, _p(w), ldw, _p(c), ldc, _s(stream)), "moss_k_gemm_nt")


def moss_k_qk_norm_rope_pack(batch, rows, n_heads, eps, qkv, q_gain, k_gain, rope, q, k, v, stream=None) -> None:
    _check(lib().moss_k_qk_norm_rope_pack(batch, rows, n_heads, eps, _p(qkv), _p(q_gain), _p(k_gain), _p(rope),
                                          _p(q), _p(k), _p(v), _s(stream)), "moss_k_qk_norm_rope_pack")


def moss_k_gemm_qkv_pack(batch, rows, n_heads, eps, a, w_qkv, q_gain, k_gain, rope, q, k, v, workspace,
                         stream=None) -> None:
    _check(lib().moss_k_gemm_qkv_pack(batch, rows, n_heads, eps, _p(a), _p(w_qkv), _p(q_gain), _p(k_gain), _p(rope),
                                      _p(q), _p(k), _p(v), _p(workspace),
                                      workspace.numel() * workspace.element_size(), _s(stream)),
           "moss_k_gemm_qkv_pack")


def moss_k_attention(batch, n_heads, rows, n_txt, txt_len, q, k, v, o, stream=None) -> None:
    _check(lib().moss_k_attention(batch, n_heads, rows, n_txt, ctypes.cast(_lens(txt_len), c_vp), _p(q), _p(k),
                                  _p(v), _p(o), _s(stream)), "moss_k_attention")


def moss_k_silu_mul(rows, mlp_inner, u, z, stream=None) -> None:
    _check(lib().moss_k_silu_mul(rows, mlp_inner, _p(u), _p(z), _s(stream)), "moss_k_silu_mul")


def moss_k_gated_add(batch, rows, d_model, h, gate, gate_stride, y, out=None, stream=None) -> None:
    _check(lib().moss_k_gated_add(batch, rows, d_model, _p(h), _p(gate), gate_stride, _p(y), _p(out), _s(stream)),
           "moss_k_gated_add")


def moss_k_gemm_silu(m, mlp_inner, k, a, lda, w_up, ldw, z, ldz, stream=None) -> None:
    _check(lib().moss_k_gemm_silu(m, mlp_inner, k, _p(a), lda, _p(w_up), ldw, _p(z), ldz, _s(stream)),
           "moss_k_gemm_silu")


def moss_k_gemm_gated_add(m, n, k, a, lda, w, ldw, h, gate, gate_stride, rows_per_item, out=None,
                          stream=None) -> None:
    _check(lib().moss_k_gemm_gated_add(m, n, k, _p(a), lda, _p(w), ldw, _p(h), _p(gate), gate_stride, rows_per_item,
                                       _p(out), _s(stream)), "moss_k_gemm_gated_add")


def moss_probe_arm(step, max_launches, every: int = 1) -> None:
    s = STEP[step] if isinstance(step, str) else int(step)
    _check(lib().moss_probe_arm(s, max_launches, every), "moss_probe_arm")


def moss_probe_collect(max_out: int = 4096) -> list:
    buf = (ctypes.c_float * max_out)()
    n = lib().moss_probe_collect(buf, max_out)
    if n < 0:
        raise MossError(-n, "moss_probe_collect")
    return [buf[i] for i in range(min(n, max_out))]
