"""Helpers of the GPU parity tests: uploads, packed layouts, metrics.

The GPU path and the oracle receive the same bf16 bits from the seeded
generator; nothing computed on the GPU is ever fed to the oracle.
"""
from __future__ import annotations

import sys

import numpy as np

from diffusion_transformer_denoiser_amd import moss
from oracle import dit_block as ob


def torch():
    import torch as t
    return t


def say(*a):
    """Print and flush, so the case is named before a GPU step runs."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(bits: np.ndarray):
    """bf16 bits (uint16) -> int16 CUDA tensor holding the same bytes."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def dev_f32(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def empty_bf16(*shape):
    t = torch()
    return t.empty(shape, dtype=t.int16, device="cuda")


def empty_f32(*shape):
    t = torch()
    return t.empty(shape, dtype=t.float32, device="cuda")


def host_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def host_f64(t) -> np.ndarray:
    """A device bf16-bits tensor -> float64 values."""
    return ob.widen_bf16(host_bits(t))


def sync():
    torch().cuda.synchronize()


# ---- packed attention layouts (as documented in include/moss.h) ----------------

def pack_qk(x_bits: np.ndarray, rows_pad: int) -> np.ndarray:
    """[B, H, T, 128] bits -> [B, H, T_pad, 128] with zero pad rows."""
    b, h, t, d = x_bits.shape
    out = np.zeros((b, h, rows_pad, d), dtype=np.uint16)
    out[:, :, :t] = x_bits
    return out


def pack_v(v_bits: np.ndarray, rows_pad: int) -> np.ndarray:
    """[B, H, T, 128] bits -> [B, H, T_pad/64, 128, 64] (per 64-key tile, transposed; zero pad keys)."""
    b, h, t, d = v_bits.shape
    full = np.zeros((b, h, rows_pad, d), dtype=np.uint16)
    full[:, :, :t] = v_bits
    tiles = full.reshape(b, h, rows_pad // 64, 64, d)  # [.., tile, key, dim]
    return np.ascontiguousarray(tiles.transpose(0, 1, 2, 4, 3))


def unpack_v(packed_bits: np.ndarray, rows: int) -> np.ndarray:
    """Inverse of pack_v: -> [B, H, T, 128] bits (and the pad keys separately)."""
    b, h, nt, d, _ = packed_bits.shape
    full = packed_bits.transpose(0, 1, 2, 4, 3).reshape(b, h, nt * 64, d)
    return full[:, :, :rows], full[:, :, rows:]


# ---- metrics ------------------------------------------------------------------------

def cos_sim(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def max_rel(a, b) -> float:
    """max|a - b| / max|b|."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / (np.max(np.abs(b)) + 1e-300))


def assert_parity(name, got, ref, cos_min=0.9997, rel_max=2e-2):
    """The acceptance bar for a floating-point output tensor: cosine and max error."""
    c, r = cos_sim(got, ref), max_rel(got, ref)
    say(f"  {name}: cos {c:.7f}  max|err|/max|ref| {r:.3e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert c >= cos_min, f"{name}: cosine {c} < {cos_min}"
    assert r <= rel_max, f"{name}: max error {r} > {rel_max}"


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^(e - 7) for |x| in [2^e, 2^(e+1)))."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_ulps(name, got, ref, ulps=1.0, abs_floor=0.0):
    """|got - ref| <= ulps * ulp_bf16(ref) + abs_floor everywhere."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    lim = ulps * bf16_ulp(ref) + abs_floor
    worst = float(np.max(err / lim))
    say(f"  {name}: worst error {worst:.3f} of the bound ({ulps} bf16 ulp + {abs_floor:g})")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert worst <= 1.0, f"{name}: error {worst:.3f} x the bound"


def geometry_dims(geom, batch=None):
    return moss.make_dims(batch or geom.batch, geom.n_img, geom.n_txt, geom.d_model, geom.mlp_inner, geom.eps)
