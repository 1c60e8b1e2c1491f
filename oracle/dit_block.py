"""Float64 oracle of one MOSS-Image-style DiT denoiser block, and a stack of them.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The GPU
library never calls it, and it shares no code with the GPU library.

What is computed, and where it is described
--------------------------------------------
The block is the one the MOSS-Image transformer page (TensorFold PR #1528,
"MOSS-Image's transformer on the CUDA runtime") lists under "What it adds":

* its four kernels: a modulated RMSNorm, q/k norm with rotary into packed
  rows, SiLU (garbled as "situ" in the page text; the encoder page, PR #1512,
  names the sibling ``me_silu_mul``), and a gated add;
* bf16 GEMM projections with fp32 sums;
* full (non-causal) attention at head dim 128 ("Shared code": the
  ``vision_kernel<128, 8>`` instance);
* the timestep's modulation, shared config code (adaLN);
* precision: bf16 weights and activations, fp32 sums, norms and softmax.

The pages do not print the block's equations.  The plain reading adopted here
(adaLN-Zero style modulation as in Peebles & Xie's DiT, the (1 + scale) form
of modulation, epsilon inside the square root, interleaved rotary pairs as in
Su et al.'s RoFormer, 2D axial rotary with y on pairs 0-31 and x on 32-63,
text rows first, SiLU-gated MLP with the gate half first, no biases) is listed
with its reasons in the design notes.

Headline mode computes every step exactly in float64 on the bf16 inputs
widened exactly.  ``rounded=True`` rounds to bf16 (to float32 for the
modulation vector and rotary tables) at each point where the GPU path stores a
tensor, as the pages' kernel contract does ("float64 at the torch code's bf16
rounding points", MOSS-Image encoder page PR #1512, "Receipt").  The residual
stream is a running sum of the blocks' gated contributions; under the fp32
sums of the precision policy it is not rounded between the gated adds or
between blocks, only when a call returns its output.  The outputs of the
out, up and down projections are consumed where they are produced (by the
gated adds and the SiLU gate) and are not rounded either.  Pages' readings
are cited per function.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# storage formats (exact widening, and rounding for the rounded mode)
# ----------------------------------------------------------------------------


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), kept in float64.

    bf16 has an 8-bit significand (7 stored bits).  ``frexp`` gives
    ``a = m * 2**e`` with ``0.5 <= |m| < 1``; rounding ``m * 2**8`` to the
    nearest integer (``rint`` rounds ties to even) keeps 8 significant bits.
    Values in bf16's subnormal range are rounded on the subnormal grid.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    e_eff = np.maximum(e, -125)  # bf16 subnormal spacing is 2**-133
    q = np.rint(np.ldexp(a, 8 - e_eff))
    return np.ldexp(q, e_eff - 8)


def round_f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def _ident(a):
    return a


# ----------------------------------------------------------------------------
# the steps
# ----------------------------------------------------------------------------


def silu(z) -> np.ndarray:
    """SiLU(z) = z / (1 + e^-z).

    MOSS-Image transformer page (PR #1528), "What it adds": the third kernel;
    the CUDA port page (PR #2281), "The kernel contract", notes that SiLU is
    not monotone and dips to about -0.278 near z = -1.278.
    """
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def rms_normalize(h, eps: float) -> np.ndarray:
    """h / sqrt(mean over the last axis of h^2 + eps), per row."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def adaln_modulation(cond, w_mod) -> np.ndarray:
    """mod = W_mod . SiLU(cond), per item: [B, D] x [6D, D] -> [B, 6D].

    MOSS-Image transformer page (PR #1528), "What it adds": the timestep's
    modulation is shared config code.  Reading: adaLN-Zero style, one linear
    map of SiLU(cond) per block, no bias; the six chunks in order are shift1,
    scale1, gate1, shift2, scale2, gate2.
    """
    return silu(cond) @ np.asarray(w_mod, dtype=np.float64).T


def split_modulation(mod, d: int) -> dict:
    names = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")
    return {n: mod[..., i * d:(i + 1) * d] for i, n in enumerate(names)}


def modulated_rmsnorm(h, shift, scale, eps: float) -> np.ndarray:
    """RMSNorm(h) * (1 + scale) + shift; no learned gain.

    MOSS-Image transformer page (PR #1528), "What it adds": the modulated
    RMSNorm kernel.
    """
    return rms_normalize(h, eps) * (1.0 + scale) + shift


def rope_tables(n_txt: int, grid_h: int, grid_w: int, theta: float = 10000.0,
                head_dim: int = 128) -> tuple:
    """2D axial rotary tables (cos, sin), each [n_txt + grid_h*grid_w, head_dim/2].

    MOSS-Image transformer page (PR #1528), "What it adds": rotary tables are
    shared config code.  Reading: text rows take angle 0 (identity); the image
    row at grid (y, x), ordered y-major after the text rows, takes angle
    y * w_i on pairs i < 32 and x * w_(i-32) on pairs i >= 32, with
    w_i = theta^(-i/32), i.e. theta^(-2i/64) for 64 dims per axis.
    """
    npair = head_dim // 2
    half = npair // 2
    w = theta ** (-np.arange(half, dtype=np.float64) / half)
    ys, xs = np.meshgrid(np.arange(grid_h, dtype=np.float64),
                         np.arange(grid_w, dtype=np.float64), indexing="ij")
    ang_img = np.concatenate([ys.reshape(-1, 1) * w[None, :], xs.reshape(-1, 1) * w[None, :]], axis=1)
    ang = np.concatenate([np.zeros((n_txt, npair)), ang_img], axis=0)
    return np.cos(ang), np.sin(ang)


def rope_rotate(x, cos, sin) -> np.ndarray:
    """Rotate interleaved pairs (x_2p, x_2p+1) of the last axis by each row's angle.

    (x_2p, x_2p+1) -> (x_2p c - x_2p+1 s, x_2p s + x_2p+1 c), c and s from the
    row's table entry for pair p.  x: [..., T, 2P]; cos, sin: [T, P].
    """
    x = np.asarray(x, dtype=np.float64)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


def qk_norm_rope(q, k, q_gain, k_gain, cos, sin, eps: float, rnd=_ident) -> tuple:
    """Per (row, head): RMSNorm over the 128 head dims times a gain, then rotary.

    q, k: [H, T, 128].  MOSS-Image transformer page (PR #1528), "What it
    adds": the "q/k norm and rotary into packed rows" kernel.  Reading: one
    gain vector for q and one for k, shared by all heads; v is not rotated.
    """
    qh = rope_rotate(rms_normalize(q, eps) * q_gain, cos, sin)
    kh = rope_rotate(rms_normalize(k, eps) * k_gain, cos, sin)
    return rnd(qh), rnd(kh)


def attention(q, k, v, key_valid, rnd=_ident) -> np.ndarray:
    """Full (non-causal) softmax attention per head; invalid keys get -inf.

    q, k, v: [H, T, hd]; key_valid: [T] bool.  S = q k^T / sqrt(hd), row
    softmax, times v.  MOSS-Image transformer page (PR #1528), "What it adds"
    and "Shared code": the full vision attention at head dim 128, with the
    softmax in fp32 per the precision bullet of "What it adds".  In rounded
    mode the probabilities are rounded to bf16 for the product with v
    (relative to the row maximum) while the normaliser sums the unrounded
    ones.
    """
    hd = q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / np.sqrt(hd)
    s = np.where(np.asarray(key_valid, dtype=bool)[None, None, :], s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = np.sum(p, axis=-1, keepdims=True)
    return (rnd(p) @ v) / l


def silu_gate(u, f: int) -> np.ndarray:
    """z = SiLU(u[:, :f]) * u[:, f:]: the SiLU-gated MLP's inner activation.

    MOSS-Image transformer page (PR #1528), "What it adds": the SiLU kernel
    between the two MLP projections.  Reading: the up projection has width
    2F with the gate half first.
    """
    return silu(u[..., :f]) * u[..., f:]


def gated_add(h, gate, y) -> np.ndarray:
    """h + gate * y: the gated residual add (PR #1528, "What it adds")."""
    return h + gate * y


# ----------------------------------------------------------------------------
# the block and the stack
# ----------------------------------------------------------------------------


def join_rows(x, txt, txt_len) -> np.ndarray:
    """h0 = [txt; x] per item, text rows first; text rows at or past txt_len are zero."""
    x = np.asarray(x, dtype=np.float64)
    txt = np.array(txt, dtype=np.float64, copy=True)
    for b, n in enumerate(txt_len):
        txt[b, int(n):, :] = 0.0
    return np.concatenate([txt, x], axis=1)


def key_mask(n_txt: int, n_img: int, txt_len) -> np.ndarray:
    """[B, T] bool: a key is valid unless it is a text row at or past txt_len."""
    m = np.ones((len(txt_len), n_txt + n_img), dtype=bool)
    for b, n in enumerate(txt_len):
        m[b, int(n):n_txt] = False
    return m


def block_residual(h0, cond, txt_len, n_txt: int, w: dict, cos, sin, eps: float,
                   rounded: bool = False, keep: bool = False):
    """One block on the joined residual rows h0 [B, T, D]; returns h2 (and steps).

    The order of the steps follows the kernels the MOSS-Image transformer page
    (PR #1528) lists under "What it adds": modulated RMSNorm, QKV projection,
    q/k norm and rotary, attention, output projection, gated add, modulated
    RMSNorm, MLP projection, SiLU, down projection, gated add.
    """
    r16 = round_bf16 if rounded else _ident
    r32 = round_f32 if rounded else _ident
    h0 = np.asarray(h0, dtype=np.float64)
    bsz, t, d = h0.shape
    hd = w["q_gain"].shape[0]
    nh = d // hd
    f = w["w_down"].shape[1]
    if rounded:
        cos, sin = round_f32(cos), round_f32(sin)
    mods = r32(adaln_modulation(cond, w["w_mod"]))  # [B, 6D]
    valid = key_mask(n_txt, t - n_txt, txt_len)
    out = np.empty_like(h0)
    steps = {k: [] for k in ("mod", "cos", "sin", "a", "qkv", "q", "k", "v", "attn", "o2", "h1", "m", "u", "z",
                             "y")}
    for b in range(bsz):
        mb = split_modulation(mods[b], d)
        a = r16(modulated_rmsnorm(h0[b], mb["shift1"], mb["scale1"], eps))
        qkv = r16(a @ w["w_qkv"].T)
        heads = qkv.reshape(t, 3, nh, hd).transpose(1, 2, 0, 3)  # [3, H, T, hd]
        q, k = qk_norm_rope(heads[0], heads[1], w["q_gain"], w["k_gain"], cos, sin, eps, r16)
        v = heads[2]
        o = r16(attention(q, k, v, valid[b], r16))
        o = o.transpose(1, 0, 2).reshape(t, d)
        o2 = o @ w["w_out"].T
        h1 = gated_add(h0[b], mb["gate1"], o2)
        m = r16(modulated_rmsnorm(h1, mb["shift2"], mb["scale2"], eps))
        u = m @ w["w_up"].T
        z = r16(silu_gate(u, f))
        y = z @ w["w_down"].T
        out[b] = gated_add(h1, mb["gate2"], y)
        if keep:
            for name, val in (("mod", mods[b]), ("cos", cos), ("sin", sin), ("a", a), ("qkv", qkv), ("q", q),
                              ("k", k), ("v", v),
                              ("attn", o), ("o2", o2), ("h1", h1), ("m", m), ("u", u), ("z", z), ("y", y)):
                steps[name].append(val)
    if keep:
        return out, {k: np.stack(v) for k, v in steps.items()}
    return out


def block_forward(x, txt, txt_len, cond, w: dict, cos, sin, eps: float = 1e-6,
                  rounded: bool = False, keep: bool = False):
    """Block output [B, n_txt + n_img, D] for image rows x and text rows txt."""
    h0 = join_rows(x, txt, txt_len)
    res = block_residual(h0, cond, txt_len, txt.shape[1], w, cos, sin, eps, rounded, keep)
    if not rounded:
        return res
    if keep:
        return round_bf16(res[0]), res[1]
    return round_bf16(res)


def stack_forward(x, txt, txt_len, cond, blocks, cos, sin, eps: float = 1e-6,
                  rounded: bool = False):
    """L blocks in sequence on the same cond and rotary tables.

    ``blocks`` is any iterable of weight dicts; a generator streams a long
    stack one block at a time.  The stack shape (many identical blocks run in
    sequence) is the transformer's; the CUDA port page (PR #2281, "What this
    changes") mentions skipping block 22 for the guidance pass, so the
    released model has more than 22 blocks.
    """
    h = join_rows(x, txt, txt_len)
    for w in blocks:
        h = block_residual(h, cond, txt_len, txt.shape[1], w, cos, sin, eps, rounded)
    return round_bf16(h) if rounded else h


def weights_f64(bits: dict) -> dict:
    """Widen a dict of bf16 weight bit arrays to float64."""
    return {k: widen_bf16(v) for k, v in bits.items()}
