"""Planted mistakes in the oracle must be caught by at least one pin (CPU only).

Each case swaps one oracle function for a copy with a plausible bug -- a wrong
index, a dropped term, a wrong sign, a transposed operand -- and checks that the
pin set fails.  This is what makes the pins worth trusting."""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as oa
import oracle.rope as orp
import oracle_pins


def _row_no_scale(q_row, K, V, scale):
    return _orig_row(q_row, K, V, 1.0)


def _row_lse_without_max(q_row, K, V, scale):
    out, lse = _orig_row(q_row, K, V, scale)
    if K.shape[0] == 0:
        return out, lse
    s = float(scale) * (np.asarray(K, np.float64) @ np.asarray(q_row, np.float64))
    return out, lse - s.max()


def _row_keys_as_values(q_row, K, V, scale):
    return _orig_row(q_row, K, K, scale)


def _row_no_normalise(q_row, K, V, scale):
    out, lse = _orig_row(q_row, K, V, scale)
    return out * math.exp(lse), lse


def _combine_wrong_sign(o_parts, lse_parts):
    return _orig_combine(o_parts, -np.asarray(lse_parts, dtype=np.float64))


def _round_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.where(np.isfinite(x), np.ldexp(np.trunc(m * 256.0), e - 8), x)


def _ulp_one_bit_short(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x > 0, x, 1.0))
    return np.ldexp(1.0, e - 7)


def _ulp_of_next_binade(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x > 0, x, 1.0))
    return np.ldexp(1.0, e - 7 - (x < 1.0))


_orig_row = oa.softmax_attention_row
_orig_combine = oa.lse_combine

MUTATIONS = {
    "gqa_modulo_mapping": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "causal_one_short": ("visible_tokens", lambda L, T, t: L - T + t),
    "causal_one_long": ("visible_tokens", lambda L, T, t: L - T + t + 2),
    "block_slot_swapped": ("block_and_slot", lambda j, bs: (j % bs, j // bs)),
    "scale_dropped": ("softmax_attention_row", _row_no_scale),
    "lse_missing_max": ("softmax_attention_row", _row_lse_without_max),
    "keys_used_as_values": ("softmax_attention_row", _row_keys_as_values),
    "missing_normalisation": ("softmax_attention_row", _row_no_normalise),
    "lse_merge_wrong_sign": ("lse_combine", _combine_wrong_sign),
    "bf16_truncates": ("round_to_bf16", _round_truncate),
    "bf16_ulp_doubled": ("bf16_ulp", _ulp_one_bit_short),
    "bf16_ulp_wrong_above_one": ("bf16_ulp", _ulp_of_next_binade),
}


def _rope_interleaved(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = orp.rope_angles(positions, D, theta)[..., None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2], y[..., 1::2] = a * c - b * s, b * c + a * s
    return y


def _rope_wrong_sign(x, positions, theta):
    return _orig_rope(x, -np.asarray(positions, dtype=np.float64), theta)


def _rope_exponent_halved(positions, D, theta):
    i = np.arange(D // 2, dtype=np.float64)
    return np.asarray(positions, dtype=np.float64)[..., None] * np.power(np.float64(theta), -i / D)


_orig_rope = orp.rope_rotate

ROPE_MUTATIONS = {
    "rope_interleaved_pairs": ("rope_rotate", _rope_interleaved),
    "rope_wrong_sign": ("rope_rotate", _rope_wrong_sign),
    "rope_exponent_halved": ("rope_angles", _rope_exponent_halved),
    "rope_position_one_late": ("token_positions", lambda lens_pre, T: np.asarray(lens_pre)[:, None]
                               + np.arange(T)[None, :] + 1),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS) + sorted(ROPE_MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name] if name in MUTATIONS else ROPE_MUTATIONS[name]
    monkeypatch.setattr(oa if name in MUTATIONS else orp, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception:  # any failure of a pin counts as caught
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
