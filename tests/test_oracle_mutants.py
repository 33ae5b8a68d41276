"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant is a one-line source edit of ``oracle/mzref.py`` (a flipped
sign, a wrong index, a dropped term, an inverted mask...).  The edited
module is executed on the CPU and swapped in for the real oracle while the
pins run; a mutant that passes every pin means the pins have a hole.
"""
import inspect
import types

import pytest

from oracle import mzref
from tests import oracle_pins

SRC = inspect.getsource(mzref)

MUTANTS = {
    "rope_sign": ("out[..., 0::2] = x0 * c - x1 * s", "out[..., 0::2] = x0 * c + x1 * s"),
    "rope_half_split": ("x0, x1 = x[..., 0::2], x[..., 1::2]", "x0, x1 = x[..., :D // 2], x[..., D // 2:]"),
    "rope_freq_no_2": ("np.power(float(base), -2.0 * i / head_dim)", "np.power(float(base), -1.0 * i / head_dim)"),
    "rope_k_unrotated": ("kh = rope(kh, pk[b], rope_base, rope_style, rope_precision, rope_factors, rope_mscale)", "kh = kh"),
    "rope_partial_off_by_one": ("min(pe_attn_head, n_heads_q)", "min(pe_attn_head + 1, n_heads_q)"),
    "gqa_modulo": ("hk = h // G", "hk = h % Hkv"),
    "scale_inverted": ("if scale <= 0:\n        scale = 1.0 / math.sqrt(D)\n    n_rot",
                       "if scale <= 0:\n        scale = math.sqrt(D)\n    n_rot"),
    "no_max_subtraction": ("m_safe = np.where(any_live, m, 0.0)", "m_safe = np.zeros_like(m)"),
    "max_over_masked": ("m = np.where(live, s, -np.inf).max(axis=1, initial=-np.inf)",
                        "m = s.max(axis=1, initial=-np.inf)"),
    "masked_keys_included": ("p = np.where(live, e, 0.0)", "p = np.where(np.isfinite(e), e, 0.0)"),
    "no_normalisation": ("(p[any_live] @ v) / l[any_live, None]", "(p[any_live] @ v)"),
    "lse_drops_max": ("m_safe + np.log(np.where(any_live, l, 1.0))", "np.log(np.where(any_live, l, 1.0))"),
    "mask_polarity": ("return np.broadcast_to(m, (B, m.shape[1], Sq, Sk))",
                      "return np.broadcast_to(~m, (B, m.shape[1], Sq, Sk))"),
    "segment_padding_attends": ("live = (sq[:, :, None] >= 0) & (sq[:, :, None] == sk[:, None, :])",
                                "live = (sq[:, :, None] == sk[:, None, :])"),
    "segment_pos_no_restart": ("            start = i\n", "            pass\n"),
    "decode_span_inclusive": ("in_span = np.arange(C) < span", "in_span = np.arange(C) <= span"),
    "decode_q_rope_dropped": ("qh = rope(qh, np.asarray(q_pos)[b], rope_base, rope_style, rope_precision, rope_factors, rope_mscale)", "qh = qh"),
    "bf16_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "fp16_bias": ("(e - 15)", "(e - 14)"),
    "fp16_subnormal": ("sub = np.ldexp(f, -24)", "sub = np.ldexp(f, -23)"),
    "empty_row_nan": ("o = np.zeros((q.shape[0], v.shape[1]))", "o = np.full((q.shape[0], v.shape[1]), np.nan)"),
    "half_split_sign": ("out[..., :D // 2] = x0 * c - x1 * s", "out[..., :D // 2] = x0 * c + x1 * s"),
    "half_split_as_interleaved": ("x0, x1 = x[..., :D // 2], x[..., D // 2:]",
                                  "x0, x1 = x[..., 0::2], x[..., 1::2]"),
    "half_split_style_ignored": ("    if style == \"half\":\n        return rope_half_split(x, pos, base, precision, factors, mscale)",
                                 "    if style == \"half\":\n        return rope_interleaved(x, pos, base, precision, factors, mscale)"),
    "causal_strict": ("live = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None]",
                      "live = np.arange(Sk)[None, :] < np.arange(Sq)[:, None]"),
    "causal_bottom_right": ("live = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None]",
                            "live = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq)"),
    "append_causal_strict": ("causal = np.arange(C)[None, :] <= pos[:, None]",
                             "causal = np.arange(C)[None, :] < pos[:, None]"),
    "append_pos_off_by_one": ("pos = L + np.arange(T)", "pos = L + 1 + np.arange(T)"),
    "append_key_unrotated": ("kr = rope(kn[b, hk], pos, rope_base, rope_style, rope_precision, rope_factors, rope_mscale) if rope_base > 0 else kn[b, hk]",
                             "kr = kn[b, hk]"),
    "append_values_not_written": ("v[b, hk, L:L + T] = vn[b, hk]", "pass"),
    "append_overflow_inclusive": ("if L < 0 or L + T > C:", "if L < 0 or L + T >= C:"),
    "longrope_factor_multiplies": ("theta = theta / np.asarray(factors, dtype=np.float64)",
                                   "theta = theta * np.asarray(factors, dtype=np.float64)"),
    "longrope_mscale_dropped": ("return np.cos(ang) * mscale, np.sin(ang) * mscale", "return np.cos(ang), np.sin(ang)"),
    "fp16_positions_exact": ("p16 = p.astype(np.float16).astype(np.float64)", "p16 = p"),
    "fp16_angle_unrounded": ("a16 = (p16 * th16).astype(np.float16).astype(np.float64)", "a16 = p16 * th16"),
    "bf16_rounding_truncates": ("r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))",
                                "r = (b >> np.uint64(16))"),
    "rms_norm_sum_not_mean": ("ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    "rms_norm_eps_outside": ("return x / np.sqrt(ms + eps) * w", "return x / (np.sqrt(ms) + eps) * w"),
    "k_norm_uses_q_weight": ("kh = rms_norm(kh, decode(k_norm_w, dtype), norm_eps)",
                             "kh = rms_norm(kh, decode(q_norm_w, dtype), norm_eps)"),
    "causal_transposed": ("live = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None]",
                          "live = np.arange(Sk)[None, :] >= np.arange(Sq)[:, None]"),
    # the parity checker (parity_stats / within_tolerance)
    "checker_or_for_and": ('return stats["rel_l2"] <= 4e-3 and stats["max_abs"]',
                           'return stats["rel_l2"] <= 4e-3 or stats["max_abs"]'),
    "checker_norm_of_out": ("nref = float(np.linalg.norm(ref))", "nref = float(np.linalg.norm(out))"),
    "checker_max_ref_of_out": ('"max_ref": float(np.abs(ref).max())', '"max_ref": float(np.abs(out).max())'),
    "checker_f32_bound_1e4": ('return stats["max_abs"] <= 1e-5', 'return stats["max_abs"] <= 1e-4'),
    "checker_f32_as_16bit": ('if dtype == "f32":\n        return stats["max_abs"] <= 1e-5',
                             'if dtype == "fp32":\n        return stats["max_abs"] <= 1e-5'),
    "checker_rel_bound_4e2": ('stats["rel_l2"] <= 4e-3', 'stats["rel_l2"] <= 4e-2'),
    "checker_abs_factor_0_2": ('stats["max_abs"] <= 2e-2 * max', 'stats["max_abs"] <= 2e-1 * max'),
    "checker_mean_abs": ('"max_abs": float(np.abs(d).max())', '"max_abs": float(np.abs(d).mean())'),
    "checker_abs_floor_1": ('max(stats["max_ref"], 1e-30)', 'max(stats["max_ref"], 1.0)'),
}


def _mutant_module(old, new):
    assert SRC.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mod = types.ModuleType("mzref_mutant")
    mod.__dict__["__name__"] = "mzref_mutant"
    exec(compile(SRC.replace(old, new), "mzref_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    monkeypatch.setattr(oracle_pins, "mzref", _mutant_module(old, new))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as e:  # noqa: BLE001 - any failure detects the mutant
            caught.append(f"{pin.__name__}: {type(e).__name__}")
            break
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_module_passes(monkeypatch):
    """The executed copy itself (no edit) passes every pin."""
    monkeypatch.setattr(oracle_pins, "mzref", _mutant_module("import math\n", "import math\n"))
    for pin in oracle_pins.ALL_PINS:
        pin()
