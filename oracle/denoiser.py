"""Float64 oracle of one whole denoiser forward: the ends around the block stack.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg may import this module.  It shares no code with the HIP path.

The pages name these parts and their sizes, not their formulas: the
timestep's modulation is shared config code (the MOSS-Image transformer page,
TensorFold PR #1528, "What it adds"); the prompt rows come from an encoder of
hidden size 4096 (the encoder page, PR #1512); the latents are rows of 128
values, 4096 of them for a 1024x1024 picture (the CUDA port page, PR #2281,
the latents.f32 files of 2,097,152 bytes).  Each part takes the standard DiT
form (Peebles & Xie, 2023), with no biases, as the blocks have none:

* timestep features: 256 values, cos(t w_i) for i < 128 then sin(t w_i),
  w_i = 10000^(-i/128) (the transformer's sinusoidal position code, cos
  half first as the DiT timestep embedder lays it out);
* cond = W_t2 SiLU(W_t1 features), rounded to bf16 as the blocks' input;
* prompt rows txt = enc W_txt^T (4096 -> D) and latent rows x = latent
  W_in^T (128 -> D), each rounded to bf16 as the stack's inputs;
* after the stack, the image rows' residual h goes through a modulated
  RMSNorm with (shift, scale) = W_fmod SiLU(cond) (the two D-wide chunks in
  that order) and the velocity is that norm's output times W_final^T
  (D -> 128).

The ``rounded`` mode rounds to bf16 where the GPU path stores bf16: cond,
the prompt and latent rows, the stack's stored intermediates (as
dit_block.block_residual does), the final norm's output and the velocity.
The residual stays unrounded through the stack, as in dit_block.
"""
from __future__ import annotations

import numpy as np

from . import dit_block as ob

N_FREQ = 256       # timestep features
LATENT_DIM = 128   # values per latent row
ENC_DIM = 4096     # encoder hidden size


def timestep_features(t, n: int = N_FREQ) -> np.ndarray:
    """[B, n] float64: cos(t w_i) for i < n/2, then sin(t w_i), w_i = 10000^(-i/(n/2))."""
    t = np.asarray(t, dtype=np.float64).reshape(-1, 1)
    half = n // 2
    w = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
    ang = t * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def timestep_cond(t, w_t1, w_t2) -> np.ndarray:
    """cond [B, D] = W_t2 SiLU(W_t1 features(t)) (float64, unrounded)."""
    f = timestep_features(t)
    return ob.silu(f @ np.asarray(w_t1, dtype=np.float64).T) @ np.asarray(w_t2, dtype=np.float64).T


def final_velocity(h_img, cond, w_fmod, w_final, eps: float, rnd=ob._ident) -> np.ndarray:
    """Velocity [B, n_img, 128] from the image rows' residual and cond."""
    d = h_img.shape[-1]
    mod = ob.silu(np.asarray(cond, dtype=np.float64)) @ np.asarray(w_fmod, dtype=np.float64).T
    shift, scale = mod[:, None, :d], mod[:, None, d:2 * d]
    a = rnd(ob.modulated_rmsnorm(h_img, shift, scale, eps))
    return rnd(a @ np.asarray(w_final, dtype=np.float64).T)


def denoiser_forward(latent, enc, txt_len, t, ends: dict, blocks, cos, sin, eps: float = 1e-6,
                     rounded: bool = False, skip=None) -> np.ndarray:
    """One denoiser forward: latent [B, n_img, 128] and encoder rows [B, n_txt, 4096]
    at timesteps t [B] -> velocity [B, n_img, 128] (float64).

    ``ends`` holds w_t1 [D, 256], w_t2 [D, D], w_txt [D, 4096], w_in [D, 128],
    w_fmod [2D, D] and w_final [128, D]; ``blocks`` the blocks' weight dicts;
    ``skip[i][b]`` true leaves item b's residual unchanged through block i."""
    rnd = ob.round_bf16 if rounded else ob._ident
    e = {k: np.asarray(v, dtype=np.float64) for k, v in ends.items()}
    cond = rnd(timestep_cond(t, e["w_t1"], e["w_t2"]))
    txt = rnd(np.asarray(enc, dtype=np.float64) @ e["w_txt"].T)
    x = rnd(np.asarray(latent, dtype=np.float64) @ e["w_in"].T)
    n_txt = txt.shape[1]
    h = ob.join_rows(x, txt, txt_len)
    for i, w in enumerate(blocks):
        if skip is None or not any(skip[i]):
            h = ob.block_residual(h, cond, txt_len, n_txt, w, cos, sin, eps, rounded)
            continue
        for b in range(h.shape[0]):
            if not skip[i][b]:
                h[b:b + 1] = ob.block_residual(h[b:b + 1], cond[b:b + 1], txt_len[b:b + 1], n_txt, w, cos, sin,
                                               eps, rounded)
    return final_velocity(h[:, n_txt:], cond, e["w_fmod"], e["w_final"], eps, rnd)
