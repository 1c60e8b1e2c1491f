"""Planted mistakes in the oracle must turn at least one pin red (CPU only).

Each mutant replaces one oracle function with a plausible wrong version (a
dropped term, a wrong sign, index or axis, swapped operands), in the manner of
the pages' planted controls that "drop or add one rounding point" and must
come out red (MOSS-Image encoder page, PR #1512, "Receipt").  The mistakes are
planted in the oracle, on the CPU; nothing here touches the GPU library.
"""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import denoiser as od
from oracle import dit_block as ob
from oracle import sampler as osm

from . import oracle_pins as P

_orig = {name: getattr(ob, name) for name in (
    "silu", "rms_normalize", "adaln_modulation", "split_modulation", "modulated_rmsnorm", "rope_tables",
    "rope_rotate", "qk_norm_rope", "attention", "silu_gate", "gated_add", "join_rows", "key_mask")}


def _silu_sign(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _rms_eps_outside(h, eps):
    h = np.asarray(h, dtype=np.float64)
    return h / (np.sqrt(np.mean(h * h, axis=-1, keepdims=True)) + eps)


def _rms_sum(h, eps):
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.sum(h * h, axis=-1, keepdims=True) + eps)


def _mod_no_silu(cond, w_mod):
    return np.asarray(cond) @ np.asarray(w_mod).T


def _split_swapped(mod, d):
    r = _orig["split_modulation"](mod, d)
    r["shift1"], r["scale1"] = r["scale1"], r["shift1"]
    return r


def _split_gates_swapped(mod, d):
    r = _orig["split_modulation"](mod, d)
    r["gate1"], r["gate2"] = r["gate2"], r["gate1"]
    return r


def _modnorm_no_one(h, shift, scale, eps):
    return ob.rms_normalize(h, eps) * scale + shift


def _rope_axes_swapped(n_txt, gh, gw, theta=10000.0, head_dim=128):
    cos, sin = _orig["rope_tables"](n_txt, gh, gw, theta, head_dim)
    h = head_dim // 4
    return (np.concatenate([cos[:, h:], cos[:, :h]], axis=1), np.concatenate([sin[:, h:], sin[:, :h]], axis=1))


def _rope_freq_wrong(n_txt, gh, gw, theta=10000.0, head_dim=128):
    return _orig["rope_tables"](n_txt, gh, gw, theta ** 2, head_dim)


def _rotate_sign(x, cos, sin):
    return _orig["rope_rotate"](x, cos, -sin)


def _rotate_half(x, cos, sin):
    x = np.asarray(x, dtype=np.float64)
    p = x.shape[-1] // 2
    x1, x2 = x[..., :p], x[..., p:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def _qk_gains_swapped(q, k, qg, kg, cos, sin, eps, rnd=lambda a: a):
    return _orig["qk_norm_rope"](q, k, kg, qg, cos, sin, eps, rnd)


def _qk_no_norm(q, k, qg, kg, cos, sin, eps, rnd=lambda a: a):
    return rnd(ob.rope_rotate(q * qg, cos, sin)), rnd(ob.rope_rotate(k * kg, cos, sin))


def _attn_no_scale(q, k, v, valid, rnd=lambda a: a):
    return _orig["attention"](q * np.sqrt(q.shape[-1]), k, v, valid, rnd)


def _attn_no_mask(q, k, v, valid, rnd=lambda a: a):
    return _orig["attention"](q, k, v, np.ones_like(valid), rnd)


def _attn_query_axis(q, k, v, valid, rnd=lambda a: a):
    s = (q @ np.swapaxes(k, -1, -2)) / np.sqrt(q.shape[-1])
    s = np.where(np.asarray(valid, dtype=bool)[None, None, :], s, -np.inf)
    p = np.exp(s - np.max(s, axis=-2, keepdims=True))
    p = np.nan_to_num(p / np.sum(p, axis=-2, keepdims=True))
    return p @ v


def _attn_k_for_v(q, k, v, valid, rnd=lambda a: a):
    return _orig["attention"](q, k, k, valid, rnd)


def _silu_gate_halves(u, f):
    return ob.silu(u[..., f:]) * u[..., :f]


def _gated_add_no_gate(h, gate, y):
    return h + y


def _join_pad_kept(x, txt, txt_len):
    return np.concatenate([np.asarray(txt, dtype=np.float64), np.asarray(x, dtype=np.float64)], axis=1)


def _key_mask_off_by_one(n_txt, n_img, txt_len):
    m = np.ones((len(txt_len), n_txt + n_img), dtype=bool)
    for b, n in enumerate(txt_len):
        m[b, int(n) + 1:n_txt] = False
    return m


MUTANTS = {
    "silu_sign": ("silu", _silu_sign),
    "rms_eps_outside_sqrt": ("rms_normalize", _rms_eps_outside),
    "rms_sum_not_mean": ("rms_normalize", _rms_sum),
    "modulation_without_silu": ("adaln_modulation", _mod_no_silu),
    "modulation_shift_scale_swapped": ("split_modulation", _split_swapped),
    "modulation_gates_swapped": ("split_modulation", _split_gates_swapped),
    "modnorm_scale_not_one_plus": ("modulated_rmsnorm", _modnorm_no_one),
    "rope_axes_swapped": ("rope_tables", _rope_axes_swapped),
    "rope_frequency_base": ("rope_tables", _rope_freq_wrong),
    "rope_sin_sign": ("rope_rotate", _rotate_sign),
    "rope_half_split_pairs": ("rope_rotate", _rotate_half),
    "qk_gains_swapped": ("qk_norm_rope", _qk_gains_swapped),
    "qk_norm_dropped": ("qk_norm_rope", _qk_no_norm),
    "attention_scale_dropped": ("attention", _attn_no_scale),
    "attention_mask_dropped": ("attention", _attn_no_mask),
    "softmax_over_queries": ("attention", _attn_query_axis),
    "attention_k_as_v": ("attention", _attn_k_for_v),
    "silu_gate_halves_swapped": ("silu_gate", _silu_gate_halves),
    "gated_add_gate_dropped": ("gated_add", _gated_add_no_gate),
    "pad_rows_not_zeroed": ("join_rows", _join_pad_kept),
    "key_mask_off_by_one": ("key_mask", _key_mask_off_by_one),
}


def _guidance_sign(v_pos, v_neg, g):
    if v_neg is None:
        return _orig_sampler["guidance"](v_pos, v_neg, g)
    return np.asarray(v_pos) + g * (np.asarray(v_neg) - np.asarray(v_pos))


def _guidance_no_base(v_pos, v_neg, g):
    if v_neg is None:
        return _orig_sampler["guidance"](v_pos, v_neg, g)
    return g * (np.asarray(v_pos) - np.asarray(v_neg))


def _euler_sign(x, v, dsigma):
    return np.asarray(x, dtype=np.float64) - dsigma * np.asarray(v, dtype=np.float64)


def _skip_ignored(x, txt, txt_len, cond, blocks, skip, cos, sin, eps=1e-6, rounded=False):
    return ob.stack_forward(x, txt, txt_len, cond, blocks, cos, sin, eps, rounded)


def _skip_other_item(x, txt, txt_len, cond, blocks, skip, cos, sin, eps=1e-6, rounded=False):
    flipped = [list(reversed(s)) for s in skip]
    return _orig_sampler["stack_forward_skip"](x, txt, txt_len, cond, blocks, flipped, cos, sin, eps, rounded)


_orig_sampler = {name: getattr(osm, name) for name in ("guidance", "euler_step", "stack_forward_skip")}

SAMPLER_MUTANTS = {
    "guidance_sign": ("guidance", _guidance_sign),
    "guidance_base_dropped": ("guidance", _guidance_no_base),
    "euler_sign": ("euler_step", _euler_sign),
    "skip_ignored": ("stack_forward_skip", _skip_ignored),
    "skip_other_item": ("stack_forward_skip", _skip_other_item),
}


def test_unmutated_oracle_passes_every_pin():
    assert P.failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ob, attr, fn)
    assert P.first_failing_pin(), f"planted mistake {name!r} passed every pin"


@pytest.mark.parametrize("name", sorted(SAMPLER_MUTANTS))
def test_sampler_mutant_is_caught(name, monkeypatch):
    attr, fn = SAMPLER_MUTANTS[name]
    monkeypatch.setattr(osm, attr, fn)
    assert P.first_failing_pin(), f"planted mistake {name!r} passed every pin"


_orig_den = {name: getattr(od, name) for name in ("timestep_features", "timestep_cond", "final_velocity")}


def _features_sin_first(t, n=256):
    f = _orig_den["timestep_features"](t, n)
    return np.concatenate([f[:, n // 2:], f[:, :n // 2]], axis=1)


def _features_base(t, n=256):
    t = np.asarray(t, dtype=np.float64).reshape(-1, 1)
    w = 10000.0 ** (-np.arange(n // 2) / n)
    return np.concatenate([np.cos(t * w), np.sin(t * w)], axis=1)


def _cond_no_silu(t, w_t1, w_t2):
    return (od.timestep_features(t) @ np.asarray(w_t1).T) @ np.asarray(w_t2).T


def _final_raw_cond(h_img, cond, w_fmod, w_final, eps, rnd=lambda a: a):
    d = h_img.shape[-1]
    mod = np.asarray(cond, dtype=np.float64) @ np.asarray(w_fmod).T
    a = rnd(ob.modulated_rmsnorm(h_img, mod[:, None, :d], mod[:, None, d:2 * d], eps))
    return rnd(a @ np.asarray(w_final).T)


def _final_shift_scale_swapped(h_img, cond, w_fmod, w_final, eps, rnd=lambda a: a):
    d = h_img.shape[-1]
    mod = ob.silu(np.asarray(cond, dtype=np.float64)) @ np.asarray(w_fmod).T
    a = rnd(ob.modulated_rmsnorm(h_img, mod[:, None, d:2 * d], mod[:, None, :d], eps))
    return rnd(a @ np.asarray(w_final).T)


DENOISER_MUTANTS = {
    "features_sin_half_first": ("timestep_features", _features_sin_first),
    "features_frequency_base": ("timestep_features", _features_base),
    "timestep_mlp_without_silu": ("timestep_cond", _cond_no_silu),
    "final_modulation_without_silu": ("final_velocity", _final_raw_cond),
    "final_shift_scale_swapped": ("final_velocity", _final_shift_scale_swapped),
}


@pytest.mark.parametrize("name", sorted(DENOISER_MUTANTS))
def test_denoiser_mutant_is_caught(name, monkeypatch):
    attr, fn = DENOISER_MUTANTS[name]
    monkeypatch.setattr(od, attr, fn)
    assert P.first_failing_pin(), f"planted mistake {name!r} passed every pin"


# ---- the rounding-point mode ----------------------------------------------------------------
# The pages' planted controls "drop or add one rounding point" (encoder page, PR #1512,
# "Receipt"); here each control is the oracle's block with one rounding point of its
# rounded mode taken out, or one added where the GPU path keeps a value unrounded.

_BLOCK_SRC = textwrap.dedent(inspect.getsource(ob.block_residual))

ROUNDING_MUTANTS = {
    # dropped
    "drop_mod_f32": ('mods = r32(adaln_modulation(cond, w["w_mod"]))', 'mods = adaln_modulation(cond, w["w_mod"])'),
    "drop_rope_f32": ("cos, sin = round_f32(cos), round_f32(sin)", "cos, sin = cos, sin"),
    "drop_a": ('a = r16(modulated_rmsnorm(h0[b], mb["shift1"], mb["scale1"], eps))',
               'a = modulated_rmsnorm(h0[b], mb["shift1"], mb["scale1"], eps)'),
    "drop_qkv": ('qkv = r16(a @ w["w_qkv"].T)', 'qkv = a @ w["w_qkv"].T'),
    "drop_qk": ('w["q_gain"], w["k_gain"], cos, sin, eps, r16)', 'w["q_gain"], w["k_gain"], cos, sin, eps, _ident)'),
    "drop_p": ("attention(q, k, v, valid[b], r16)", "attention(q, k, v, valid[b], _ident)"),
    "drop_attn_out": ("o = r16(attention(q, k, v, valid[b], r16))", "o = attention(q, k, v, valid[b], r16)"),
    "drop_m": ('m = r16(modulated_rmsnorm(h1, mb["shift2"], mb["scale2"], eps))',
               'm = modulated_rmsnorm(h1, mb["shift2"], mb["scale2"], eps)'),
    "drop_z": ("z = r16(silu_gate(u, f))", "z = silu_gate(u, f)"),
    # added
    "add_o2": ('o2 = o @ w["w_out"].T', 'o2 = r16(o @ w["w_out"].T)'),
    "add_h1": ('h1 = gated_add(h0[b], mb["gate1"], o2)', 'h1 = r16(gated_add(h0[b], mb["gate1"], o2))'),
    "add_u": ('u = m @ w["w_up"].T', 'u = r16(m @ w["w_up"].T)'),
    "add_y": ('y = z @ w["w_down"].T', 'y = r16(z @ w["w_down"].T)'),
    "add_out": ('out[b] = gated_add(h1, mb["gate2"], y)', 'out[b] = r16(gated_add(h1, mb["gate2"], y))'),
}


def _mutated_block(old, new):
    assert _BLOCK_SRC.count(old) == 1, f"the control's text must occur once in block_residual: {old!r}"
    ns = dict(vars(ob))
    exec(compile(_BLOCK_SRC.replace(old, new), "<planted control>", "exec"), ns)  # noqa: S102
    return ns["block_residual"]


@pytest.mark.parametrize("name", sorted(ROUNDING_MUTANTS))
def test_rounding_point_control_is_caught(name, monkeypatch):
    monkeypatch.setattr(ob, "block_residual", _mutated_block(*ROUNDING_MUTANTS[name]))
    assert P.first_failing_pin(), f"planted control {name!r} passed every pin"


def _qk_unrounded(q, k, qg, kg, cos, sin, eps, rnd=lambda a: a):
    return _orig["qk_norm_rope"](q, k, qg, kg, cos, sin, eps)


def test_qk_left_unrounded_is_caught(monkeypatch):
    """q and k not stored in bf16 in the rounded mode (the q/k kernel's own rounding point)."""
    monkeypatch.setattr(ob, "qk_norm_rope", _qk_unrounded)
    assert P.first_failing_pin(), "q/k left unrounded passed every pin"


def test_denoiser_skip_other_item_is_caught(monkeypatch):
    """The skip table applied to the other item of the guidance pair."""
    orig = od.denoiser_forward

    def flipped(*args, skip=None, **kw):
        return orig(*args, skip=[list(reversed(r)) for r in skip] if skip is not None else None, **kw)

    monkeypatch.setattr(od, "denoiser_forward", flipped)
    assert P.first_failing_pin(), "skip applied to the other item passed every pin"


def test_rounding_controls_change_the_rounded_output(monkeypatch):
    """Each control really changes what the rounded mode computes (so catching it means something):
    a step of one block, or the output of a 2-block rounded stack (a rounding of the residual
    between blocks is invisible in one block, whose output is rounded anyway)."""
    geom = P.tiny_geoms()[1]
    x, txt, lens, cond, ws = P.f64_inputs(geom, seed=6, n_blocks=2)
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    _, base = ob.block_forward(x, txt, lens, cond, ws[0], cos, sin, geom.eps, rounded=True, keep=True)
    stack = ob.stack_forward(x, txt, lens, cond, ws, cos, sin, geom.eps, rounded=True)
    for name, (old, new) in ROUNDING_MUTANTS.items():
        monkeypatch.setattr(ob, "block_residual", _mutated_block(old, new))
        _, st = ob.block_forward(x, txt, lens, cond, ws[0], cos, sin, geom.eps, rounded=True, keep=True)
        changed = any(not np.array_equal(st[k], base[k]) for k in base)
        changed |= not np.array_equal(ob.stack_forward(x, txt, lens, cond, ws, cos, sin, geom.eps, rounded=True), stack)
        assert changed, name
