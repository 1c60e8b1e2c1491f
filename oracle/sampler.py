"""Float64 oracle of the sampler step around the denoiser stack.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg may import this module.  It shares no code with the HIP path.

What it computes (the MOSS-Image CUDA port page, TensorFold PR #2281, "What
this changes": the host runs the pipeline's schedule, noise and classifier-free
guidance with an empty negative prompt, block 22 skipped, and guidance 1
skipping the negative pass; the transformer page, PR #1528, "Measured": 50
Euler steps at guidance 3).  The pages name the pieces, not the formulas, so
this takes the standard ones:

* guidance: v = v_neg + g * (v_pos - v_neg), the classifier-free guidance
  combination (Ho & Salimans, 2022); at g = 1 it is v_pos and the negative
  pass is not needed at all;
* one explicit Euler step of the flow ODE dx/dsigma = v: x <- x + dsigma * v,
  dsigma = sigma_next - sigma_now (negative while denoising);
* a skipped block is a block that is not applied: that item's residual passes
  through it unchanged, while the other items of the batch run it.
"""
from __future__ import annotations

import numpy as np

from . import dit_block as ob


def guidance(v_pos, v_neg, g: float) -> np.ndarray:
    """Classifier-free guidance of two velocity fields (float64).

    ``v_neg`` None means the negative pass was skipped, which is only right
    at g = 1."""
    v_pos = np.asarray(v_pos, dtype=np.float64)
    if v_neg is None:
        if g != 1.0:
            raise ValueError("the negative pass can be skipped only at guidance 1")
        return v_pos
    v_neg = np.asarray(v_neg, dtype=np.float64)
    return v_neg + g * (v_pos - v_neg)


def euler_step(x, v, dsigma: float) -> np.ndarray:
    """x + dsigma * v: one explicit Euler step of dx/dsigma = v."""
    return np.asarray(x, dtype=np.float64) + dsigma * np.asarray(v, dtype=np.float64)


def guidance_euler(x, v_pos, v_neg, g: float, dsigma: float) -> np.ndarray:
    """One sampler step: guide the two velocities, then step the latent."""
    return euler_step(x, guidance(v_pos, v_neg, g), dsigma)


def stack_forward_skip(x, txt, txt_len, cond, blocks, skip, cos, sin, eps: float = 1e-6,
                       rounded: bool = False):
    """The block stack with some blocks not applied to some items.

    ``blocks`` is a list of weight dicts; ``skip[i][b]`` true means block i
    leaves item b's residual unchanged.  Items are independent (attention is
    per item), so each item runs its own list of blocks."""
    n_txt = txt.shape[1]
    outs = []
    for b in range(x.shape[0]):
        h = ob.join_rows(x[b:b + 1], txt[b:b + 1], txt_len[b:b + 1])
        for i, w in enumerate(blocks):
            if skip[i][b]:
                continue
            h = ob.block_residual(h, cond[b:b + 1], txt_len[b:b + 1], n_txt, w, cos, sin, eps, rounded)
        outs.append(h[0])
    h = np.stack(outs)
    return ob.round_bf16(h) if rounded else h
