"""Seeded synthetic inputs for the DiT denoiser block: shapes, seeds, bf16 bits.

This module holds no arithmetic of the block itself. It draws normal variates,
scales them, and stores them as bfloat16 bit patterns (uint16). Both the GPU
path and the float64 oracle receive exactly these bits.

Recipe (every draw is reproducible from ``seed`` alone, independent of the
number of threads used to make it):

* Each tensor has its own stream, ``SeedSequence(seed, spawn_key=key)`` with
  ``key = (0, t)`` for activation tensor ``t`` (0 = x, 1 = txt, 2 = cond, 3+ =
  extra test tensors) and ``key = (1 + block, j)`` for weight ``j`` of a block
  (0 = w_mod, 1 = w_qkv, 2 = q_gain, 3 = k_gain, 4 = w_out, 5 = w_up,
  6 = w_down).
* A tensor is drawn in chunks of ``CHUNK`` values in row-major order; chunk
  ``c`` comes from a PCG64 seeded with ``key + (c,)``.
* Each chunk is ``standard_normal`` in float32, multiplied by the tensor's
  standard deviation in float32 (and 1.0 added for the q/k gains), then
  rounded to bfloat16 with round-to-nearest-even.
* Text rows at or beyond an item's ``txt_len`` are zero.

The shapes follow the pages' workloads: text rows of 34, 63 and 10 (the fox,
sticky-note and empty prompts of the MOSS-Image encoder page, "Receipt"), and
image grids of 64x64 (1024x1024 picture) and 75x55 (1200x880 picture) at one
token per 16x16 pixel patch (MOSS-Image transformer on CUDA, "Measured").
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

CHUNK = 1 << 24
WEIGHT_STD = 0.02
ACT_STD = 1.0

WEIGHT_NAMES = ("w_mod", "w_qkv", "q_gain", "k_gain", "w_out", "w_up", "w_down")


@dataclass(frozen=True)
class Geometry:
    """One workload: batch, rows, widths.  Rows are text first, then image."""

    name: str
    batch: int
    n_txt: int
    grid_h: int
    grid_w: int
    d_model: int
    n_heads: int
    mlp_inner: int
    head_dim: int = 128
    eps: float = 1e-6
    theta: float = 10000.0
    txt_len: tuple = field(default=())
    n_blocks: int = 1

    @property
    def n_img(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def rows(self) -> int:
        return self.n_txt + self.n_img

    def lengths(self) -> tuple:
        return self.txt_len if self.txt_len else (self.n_txt,) * self.batch

    def block_flops(self) -> float:
        """Dense multiply-add work of one block forward, 2 flops per MAC.

        Counts the padded rows the GPU computes (all ``batch * rows``); the
        attention term counts every query against every key of its item.
        """
        m = self.batch * self.rows
        d, f = self.d_model, self.mlp_inner
        gemm = 2.0 * m * d * (3 * d + d + 2 * f) + 2.0 * m * f * d
        attn = 2.0 * 2.0 * self.batch * self.n_heads * self.rows * self.rows * self.head_dim
        gemv = 2.0 * self.batch * 6 * d * d
        return gemm + attn + gemv


CONFIGS = {
    # small case: D=256 (2 heads), MLP 1024, 8x8 grid + 8 text rows
    "c0": Geometry("c0", 1, 8, 8, 8, 256, 2, 1024),
    # D=3072 (24 heads), MLP 12288, 32x32 grid + 34 text rows
    "c1": Geometry("c1", 1, 34, 32, 32, 3072, 24, 12288),
    # 1024x1024 picture: 64x64 grid + 34 text rows
    "c2": Geometry("c2", 1, 34, 64, 64, 3072, 24, 12288),
    # 1200x880 picture: 75 wide x 55 high + 63 text rows (ragged tiles)
    "c3": Geometry("c3", 1, 63, 55, 75, 3072, 24, 12288),
    # 24-block stack, two guidance items: 34 and 10 valid text rows
    "c4": Geometry("c4", 2, 34, 64, 64, 3072, 24, 12288, txt_len=(34, 10), n_blocks=24),
    # larger pictures, 16 pixels per latent row (1280x1024, 1408x1024, 1536x1024 wide x high)
    "p1280": Geometry("p1280", 1, 34, 64, 80, 3072, 24, 12288),
    "p1408": Geometry("p1408", 1, 34, 64, 88, 3072, 24, 12288),
    "p1536": Geometry("p1536", 1, 34, 64, 96, 3072, 24, 12288),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed: int, key: tuple, shape: tuple, std: float, offset: float = 0.0) -> np.ndarray:
    """bf16 bits of ``offset + std * N(0, 1)`` drawn from stream ``key``."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK
    std32 = np.float32(std)
    off32 = np.float32(offset)

    def one(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        ss = np.random.SeedSequence(seed, spawn_key=tuple(key) + (c,))
        g = np.random.Generator(np.random.PCG64(ss))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        v *= std32
        if offset != 0.0:
            v += off32
        out[lo:hi] = f32_to_bf16_bits(v)

    if nchunks <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunks)))
    return out.reshape(shape)


def make_activations(geom: Geometry, seed: int = 0) -> dict:
    """x [B, n_img, D], txt [B, n_txt, D] (pad rows zero), txt_len int32 [B], cond [B, D]."""
    b, d = geom.batch, geom.d_model
    x = normal_bf16(seed, (0, 0), (b, geom.n_img, d), ACT_STD)
    txt = normal_bf16(seed, (0, 1), (b, geom.n_txt, d), ACT_STD)
    lens = np.asarray(geom.lengths(), dtype=np.int32)
    for i, n in enumerate(lens):
        txt[i, n:, :] = 0
    cond = normal_bf16(seed, (0, 2), (b, d), ACT_STD)
    return {"x": x, "txt": txt, "txt_len": lens, "cond": cond}


def make_block_weights(geom: Geometry, seed: int = 0, block: int = 0, std: float = WEIGHT_STD,
                       gain_std: float = WEIGHT_STD, gain_mean: float = 1.0) -> dict:
    """Weights of one block as bf16 bits; projection matrices are row-major [out, in].

    ``std`` defaults to the workloads' N(0, 0.02).  A small geometry drawn with
    ``std = 0.02 * sqrt(3072 / d_model)`` has the same branch magnitudes as the
    D = 3072 block (each projection output's spread scales with std * sqrt(D)).
    ``gain_mean`` scales the q/k gains (4.0 makes the logits about N(0, 16)).
    """
    d, f, hd = geom.d_model, geom.mlp_inner, geom.head_dim
    k = 1 + block
    return {
        "w_mod": normal_bf16(seed, (k, 0), (6 * d, d), std),
        "w_qkv": normal_bf16(seed, (k, 1), (3 * d, d), std),
        "q_gain": normal_bf16(seed, (k, 2), (hd,), gain_std, offset=gain_mean),
        "k_gain": normal_bf16(seed, (k, 3), (hd,), gain_std, offset=gain_mean),
        "w_out": normal_bf16(seed, (k, 4), (d, d), std),
        "w_up": normal_bf16(seed, (k, 5), (2 * f, d), std),
        "w_down": normal_bf16(seed, (k, 6), (d, f), std),
    }


def normal_f32(seed: int, key: tuple, shape: tuple, std: float) -> np.ndarray:
    """float32 values ``std * N(0, 1)`` from stream ``key`` (no bf16 rounding)."""
    n = int(np.prod(shape)) if len(shape) else 1
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key) + (0,))))
    v = g.standard_normal(n, dtype=np.float32)
    v *= np.float32(std)
    return v.reshape(shape)


LATENT_DIM = 128   # values per latent row
ENC_DIM = 4096     # prompt encoder hidden size
END_NAMES = ("w_t1", "w_t2", "w_txt", "w_in", "w_fmod", "w_final")


def make_ends_weights(geom: Geometry, seed: int = 0, enc_dim: int = ENC_DIM, std: float = WEIGHT_STD) -> dict:
    """The denoiser's end weights as bf16 bits, row-major [out, in]: the timestep
    MLP w_t1 [D, 256] and w_t2 [D, D], the prompt projection w_txt [D, enc_dim],
    the latent projection w_in [D, 128], the final modulation w_fmod [2D, D] and
    the final projection w_final [128, D]; stream group 1000."""
    d = geom.d_model
    shapes = {"w_t1": (d, 256), "w_t2": (d, d), "w_txt": (d, enc_dim), "w_in": (d, LATENT_DIM),
              "w_fmod": (2 * d, d), "w_final": (LATENT_DIM, d)}
    return {name: normal_bf16(seed, (1000, j), shapes[name], std) for j, name in enumerate(END_NAMES)}


def make_denoiser_inputs(geom: Geometry, seed: int = 0, enc_dim: int = ENC_DIM) -> dict:
    """latent [B, n_img, 128] and prompt rows enc [B, n_txt, enc_dim] (bf16 bits,
    N(0, 1); pad rows zero), txt_len [B], timesteps t [B] float32 in [0, 1000)."""
    b = geom.batch
    latent = normal_bf16(seed, (2000, 0), (b, geom.n_img, LATENT_DIM), ACT_STD)
    enc = normal_bf16(seed, (2000, 1), (b, geom.n_txt, enc_dim), ACT_STD)
    lens = np.asarray(geom.lengths(), dtype=np.int32)
    for i, n in enumerate(lens):
        enc[i, n:, :] = 0
    t = np.array([1000.0 * ((0.37 * seed + 0.13 + 0.29 * i) % 1.0) for i in range(b)], dtype=np.float32)
    return {"latent": latent, "enc": enc, "txt_len": lens, "t": t}


def make_tensor(seed: int, tag: int, shape: tuple, std: float = 1.0) -> np.ndarray:
    """An extra test tensor (bf16 bits) on activation stream ``(0, 3 + tag)``."""
    return normal_bf16(seed, (0, 3 + tag), shape, std)


def smaller(geom: Geometry, **kw) -> Geometry:
    return replace(geom, **kw)
