"""Pure-Python, loop-only twin of the block oracle, for tiny inputs.

TEST INFRASTRUCTURE.  Only ``tests/`` may import this module.

It is written independently of ``dit_block`` so that the two pin each other:
every product is an explicit loop, the rotary step multiplies complex numbers
``(x_2p + i x_2p+1) * e^(i angle)`` instead of applying a 2x2 rotation, the
rotary angles come from grid positions here rather than from ``rope_tables``,
and softmax is an explicit max / exp / sum over each query's keys.  The
computation is the block the MOSS-Image transformer page (TensorFold PR #1528,
"What it adds") describes, under the readings stated in ``dit_block``.

The ``rounded`` mode stores each intermediate the way the GPU path does (the
encoder page, PR #1512, "Receipt": float64 at the bf16 rounding points): the
modulation vector and the rotary cos/sin in float32, the norm outputs, the
projection output qkv, the normed and rotated q and k, the softmax weights
that multiply v (the normaliser sums the unrounded ones), the attention
output and the SiLU-gated activation in bf16, the block output in bf16.  The
residual and the out, up and down projection sums stay unrounded.  Its
rounding is its own: bf16 round-to-nearest-even on the float64 bit pattern
(drop 45 mantissa bits, round half to even on the dropped part) and float32
through ``struct``, not the NumPy ``frexp`` / ``astype`` of ``dit_block``.
"""
from __future__ import annotations

import cmath
import math
import struct
from operator import mul


def bf16(x: float) -> float:
    """Round a float to the nearest bf16 value, ties to even, on its float64 bits.

    bf16 keeps 7 of float64's 52 stored mantissa bits: the low 45 are dropped and
    the kept part goes up by one when the dropped part is over half, or exactly
    half with the kept part odd (a carry into the exponent is the right result).
    Below bf16's smallest normal (2^-126) the spacing is fixed at 2^-133."""
    if x == 0.0 or not math.isfinite(x):
        return x
    if abs(x) < 2.0 ** -126:
        return round(x * 2.0 ** 133) * 2.0 ** -133  # round() on floats: half to even
    bits = struct.unpack("<Q", struct.pack("<d", x))[0]
    drop = 45
    rest = bits & ((1 << drop) - 1)
    kept = bits >> drop
    half = 1 << (drop - 1)
    if rest > half or (rest == half and kept & 1):
        kept += 1
    return struct.unpack("<d", struct.pack("<Q", kept << drop))[0]


def f32(x: float) -> float:
    """Round a float to the nearest float32 value (struct packs with IEEE round to nearest)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _same(x: float) -> float:
    return x


def _dot(a, b) -> float:
    return math.fsum(map(mul, a, b))


def _matvec_rows(rows, w):
    """rows [n][k] times w[o][k]^T -> [n][o]."""
    return [[_dot(r, wo) for wo in w] for r in rows]


def _silu(z: float) -> float:
    if z < -700.0:
        return 0.0
    return z / (1.0 + math.exp(-z))


def _rms(row, eps: float):
    ms = math.fsum(v * v for v in row) / len(row)
    inv = 1.0 / math.sqrt(ms + eps)
    return [v * inv for v in row]


def positions(n_txt: int, grid_h: int, grid_w: int):
    """(y, x) grid position per row; text rows sit at (0, 0)."""
    pos = [(0, 0)] * n_txt
    for y in range(grid_h):
        for x in range(grid_w):
            pos.append((y, x))
    return pos


def angles(pos, theta: float, head_dim: int):
    """Rotary angle per (row, pair): y-axis frequencies on the first half of pairs."""
    half = head_dim // 4
    out = []
    for (y, x) in pos:
        row = []
        for p in range(head_dim // 2):
            if p < half:
                row.append(y * theta ** (-p / half))
            else:
                row.append(x * theta ** (-(p - half) / half))
        out.append(row)
    return out


def _rotate(vec, rot_row):
    """Multiply each pair (x_2p + i x_2p+1) by its unit complex number rot_row[p]."""
    out = []
    for p, e in enumerate(rot_row):
        z = complex(vec[2 * p], vec[2 * p + 1]) * e
        out.extend((z.real, z.imag))
    return out


def block(x, txt, txt_len, cond, w, ang, eps: float, rounded: bool = False, steps=None):
    """One block for nested-list inputs.

    x [B][n_img][D], txt [B][n_txt][D], txt_len [B], cond [B][D]; w holds
    nested lists ``w_mod [6D][D]``, ``w_qkv [3D][D]``, ``q_gain [128]``,
    ``k_gain [128]``, ``w_out [D][D]``, ``w_up [2F][D]``, ``w_down [D][F]``;
    ang [T][64] rotary angles.  Returns the block output [B][T][D] (rounded to
    bf16 in rounded mode).  With ``steps`` (a dict), each item's intermediates
    are appended to steps[name] (names as in ``dit_block``)."""
    hd = len(w["q_gain"])
    out = []
    for b in range(len(x)):
        n_txt = len(txt[b])
        rows = [list(r) if i < txt_len[b] else [0.0] * len(r) for i, r in enumerate(txt[b])]
        rows += [list(r) for r in x[b]]
        res = block_rows(rows, txt_len[b], n_txt, cond[b], w, ang, eps, hd, rounded, steps)
        out.append([[bf16(v) for v in r] for r in res] if rounded else res)
    return out


def block_rows(h0, n_valid_txt: int, n_txt: int, cond_b, w, ang, eps: float, hd: int,
               rounded: bool = False, steps=None):
    r16 = bf16 if rounded else _same
    r32 = f32 if rounded else _same
    d = len(h0[0])
    t = len(h0)
    nh = d // hd
    f = len(w["w_down"][0])
    s = [_silu(c) for c in cond_b]
    mod = [r32(_dot(wr, s)) for wr in w["w_mod"]]
    shift1, scale1, gate1 = mod[0:d], mod[d:2 * d], mod[2 * d:3 * d]
    shift2, scale2, gate2 = mod[3 * d:4 * d], mod[4 * d:5 * d], mod[5 * d:6 * d]

    a = [[r16(n * (1.0 + sc) + sh) for n, sc, sh in zip(_rms(r, eps), scale1, shift1)] for r in h0]
    qkv = [[r16(v) for v in row] for row in _matvec_rows(a, w["w_qkv"])]
    key_ok = [not (n_valid_txt <= j < n_txt) for j in range(t)]
    o = [[0.0] * d for _ in range(t)]
    qh, kh = [], []
    # the rotary tables as applied (float32-stored in rounded mode): e^(i a) per row and pair
    rot = [[cmath.exp(1j * av) for av in row] for row in ang[:t]]
    if rounded:
        rot = [[complex(r32(e.real), r32(e.imag)) for e in row] for row in rot]
    inv_sqrt = 1.0 / math.sqrt(hd)
    for e in range(nh):
        qs, ks, vs = [], [], []
        for r in range(t):
            q = qkv[r][e * hd:(e + 1) * hd]
            k = qkv[r][d + e * hd:d + (e + 1) * hd]
            v = qkv[r][2 * d + e * hd:2 * d + (e + 1) * hd]
            q = [g * val for g, val in zip(w["q_gain"], _rms(q, eps))]
            k = [g * val for g, val in zip(w["k_gain"], _rms(k, eps))]
            qs.append([r16(val) for val in _rotate(q, rot[r])])
            ks.append([r16(val) for val in _rotate(k, rot[r])])
            vs.append(v)
        qh.append(qs)
        kh.append(ks)
        for i in range(t):
            scores = [(_dot(qs[i], ks[j]) * inv_sqrt if key_ok[j] else None) for j in range(t)]
            mx = max(sv for sv in scores if sv is not None)
            ps = [(math.exp(sv - mx) if sv is not None else 0.0) for sv in scores]
            tot = math.fsum(ps)
            pr = [r16(pv) for pv in ps]  # the weights that multiply v
            for c in range(hd):
                o[i][e * hd + c] = r16(math.fsum(pr[j] * vs[j][c] for j in range(t)) / tot)
    o2 = _matvec_rows(o, w["w_out"])
    h1 = [[hv + g * ov for hv, g, ov in zip(hr, gate1, orow)] for hr, orow in zip(h0, o2)]
    m = [[r16(n * (1.0 + sc) + sh) for n, sc, sh in zip(_rms(r, eps), scale2, shift2)] for r in h1]
    u = _matvec_rows(m, w["w_up"])
    z = [[r16(_silu(ur[c]) * ur[f + c]) for c in range(f)] for ur in u]
    y = _matvec_rows(z, w["w_down"])
    h2 = [[hv + g * yv for hv, g, yv in zip(hr, gate2, yr)] for hr, yr in zip(h1, y)]
    if steps is not None:
        for name, val in (("mod", mod), ("cos", [[e.real for e in row] for row in rot]),
                          ("sin", [[e.imag for e in row] for row in rot]), ("a", a), ("qkv", qkv), ("q", qh),
                          ("k", kh), ("attn", o), ("o2", o2),
                          ("h1", h1), ("m", m), ("u", u), ("z", z), ("y", y)):
            steps.setdefault(name, []).append(val)
    return h2


def denoiser(latent, enc, txt_len, t, ends, blocks, ang, eps: float, skip=None, rounded: bool = False):
    """The whole denoiser forward for nested-list inputs, loop by loop.

    latent [B][n_img][128], enc [B][n_txt][E], t [B]; ends holds nested lists
    w_t1 [D][256], w_t2 [D][D], w_txt [D][E], w_in [D][128], w_fmod [2D][D],
    w_final [128][D]; blocks is a list of block weight dicts as for ``block``;
    ``skip[i][b]`` true passes item b's rows through block i untouched.
    Returns the velocity [B][n_img][128].  Same readings as oracle.denoiser;
    the frequencies come from math.pow and each feature is built one at a time.
    In rounded mode cond, the prompt and latent rows, the final norm's output
    and the velocity are stored in bf16, and the blocks run in rounded mode."""
    r16 = bf16 if rounded else _same
    out = []
    for b in range(len(latent)):
        feats = []
        for i in range(256):
            w_i = math.pow(10000.0, -(i % 128) / 128.0)
            feats.append(math.cos(t[b] * w_i) if i < 128 else math.sin(t[b] * w_i))
        hid = [_silu(v) for v in _matvec_rows([feats], ends["w_t1"])[0]]
        cond = [r16(v) for v in _matvec_rows([hid], ends["w_t2"])[0]]
        txt_rows = [[r16(v) for v in r] for r in _matvec_rows(enc[b], ends["w_txt"])]
        x_rows = [[r16(v) for v in r] for r in _matvec_rows(latent[b], ends["w_in"])]
        n_txt = len(txt_rows)
        rows = [list(r) if i < txt_len[b] else [0.0] * len(r) for i, r in enumerate(txt_rows)] + x_rows
        for i, w in enumerate(blocks):
            if skip is not None and skip[i][b]:
                continue
            rows = block_rows(rows, txt_len[b], n_txt, cond, w, ang, eps, len(w["q_gain"]), rounded)
        d = len(cond)
        s = [_silu(v) for v in cond]
        mod = _matvec_rows([s], ends["w_fmod"])[0]
        shift, scale = mod[:d], mod[d:2 * d]
        normed = [[r16(v * (1.0 + scale[j]) + shift[j]) for j, v in enumerate(_rms(r, eps))] for r in rows[n_txt:]]
        out.append([[r16(v) for v in r] for r in _matvec_rows(normed, ends["w_final"])])
    return out
