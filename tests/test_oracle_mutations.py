"""Planted mistakes in the oracle must each trip at least one pin.

Every mutant below is a plausible slip (a dropped term, a wrong sign, index,
scale or operand).  It is patched into the oracle module for the duration of
one test only, on the CPU, and the whole pin set is run against it.
"""

import math

import numpy as np
import pytest

import oracle.mla_oracle as O
from oracle_pins import ALL_PINS

F64 = np.float64


def _rope_neg(x, pos, base):
    x = np.asarray(x, F64)
    d = x.shape[-1]
    ang = np.asarray(pos, F64)[..., None] * O.rope_inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)))
    out[..., 0::2] = x1 * c + x2 * s
    out[..., 1::2] = -x1 * s + x2 * c
    return out


def _rope_half_split(x, pos, base):
    x = np.asarray(x, F64)
    d = x.shape[-1]
    ang = np.asarray(pos, F64)[..., None] * O.rope_inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def _inv_freq_half(d_r, base):
    i = np.arange(d_r // 2, dtype=F64)
    return np.power(F64(base), -i / d_r)


_real_attention = O.attention


def _attention_scale_dk(q_c, q_r, q_pos, cache, w_uk, w_uv, d_c, scale=None, base=10000.0, key_range=None, heads=None):
    return _real_attention(q_c, q_r, q_pos, cache, w_uk, w_uv, d_c, 1.0 / math.sqrt(np.asarray(q_c).shape[1]),
                           base, key_range, heads)


def _attention_scale_dc(q_c, q_r, q_pos, cache, w_uk, w_uv, d_c, scale=None, base=10000.0, key_range=None, heads=None):
    return _real_attention(q_c, q_r, q_pos, cache, w_uk, w_uv, d_c,
                           1.0 / math.sqrt(d_c + np.asarray(q_r).shape[1]), base, key_range, heads)


def _softmax_lse_no_max(s):
    if s.size == 0:
        return s.copy(), -math.inf
    m = np.max(s)
    e = np.exp(s - m)
    return e / e.sum(), float(math.log(e.sum()))


def _merge_unnormalised(parts, lses):
    parts = np.asarray(parts, F64)
    lses = np.asarray(lses, F64)
    m = np.max(lses, axis=0)
    w = np.where(np.isfinite(lses), np.exp(lses - np.where(np.isfinite(m), m, 0)[None]), 0.0)
    return np.einsum("sh,shd->hd", w, parts), np.where(np.isfinite(m), m + np.log(w.sum(0)), -math.inf)


def _gather_wrong(pool, table, b, length):
    page = pool.shape[1]
    out = np.empty((length, pool.shape[2]), dtype=pool.dtype)
    for t0 in range(0, length, page):
        n = min(page, length - t0)
        out[t0:t0 + n] = pool[int(table[b, 0]) if t0 else int(table[b, 0]), :n]
    return out


def _e4m3_decode_bias8(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, (c & 7).astype(F64)
    mag = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * np.exp2((e - 8).astype(F64)))
    return np.where((c & 0x7F) == 0x7F, np.nan, np.where(c & 0x80, -mag, mag))


_real_encode = O.e4m3_encode


def _e4m3_encode_truncating(x):
    x = np.asarray(x, F64)
    lo = _real_encode(x)
    # step toward zero where the nearest code lies above the magnitude
    over = np.abs(O.e4m3_decode(lo)) > np.abs(x)
    return np.where(over & ((lo & 0x7F) > 0), lo - 1, lo).astype(np.uint8)


def _scale_exponent_floor(amax):
    amax = np.asarray(amax, F64)
    return np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 0).astype(np.int64)


def _rms_sum_not_mean(c, eps=1e-6):
    c = np.asarray(c, F64)
    return c / np.sqrt(np.sum(c * c, axis=-1, keepdims=True) + eps)


def _rms_eps_outside_sqrt(c, eps=1e-6):
    c = np.asarray(c, F64)
    return c / (np.sqrt(np.mean(c * c, axis=-1, keepdims=True)) + eps)


def _rms_multiplies(c, eps=1e-6):
    c = np.asarray(c, F64)
    return c * np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)


def _rms_wrong_axis(c, eps=1e-6):
    c = np.asarray(c, F64)
    return c / np.sqrt(np.mean(c * c, axis=0, keepdims=True) + eps)


MUTANTS = {
    "precompose_query_untransposed_key": ("precompose_query_weights", lambda uq, uk: np.einsum(
        "hqk,hkc->hqc", np.asarray(uq, F64), np.asarray(uk, F64).reshape(uk.shape[0], uk.shape[2], uk.shape[1]))),
    "precompose_out_wrong_head_rows": ("precompose_out_weights", lambda uv, wo: np.einsum(
        "hcv,hvm->hcm", np.asarray(uv, F64), np.roll(np.asarray(wo, F64).reshape(uv.shape[0], uv.shape[2], -1), 1, 0))),
    "fused_output_drops_a_head": ("out_proj_fused", lambda z, w: np.einsum(
        "...hc,hcm->...m", np.asarray(z, F64)[..., 1:, :], np.asarray(w, F64)[1:])),
    "e4m3_exponent_bias_8": ("e4m3_decode", _e4m3_decode_bias8),
    "e4m3_truncates": ("e4m3_encode", _e4m3_encode_truncating),
    "fp8_scale_rounds_down": ("fp8_scale_exponent", _scale_exponent_floor),
    "rope_opposite_sign": ("rope", _rope_neg),
    "rope_half_split_pairs": ("rope", _rope_half_split),
    "rope_frequency_exponent": ("rope_inv_freq", _inv_freq_half),
    "score_drops_position_term": ("score_row", lambda qc, qr, K, kr, sc: (K @ qc) * sc),
    "score_drops_content_term": ("score_row", lambda qc, qr, K, kr, sc: (kr @ qr) * sc),
    "scale_sqrt_dk": ("attention", _attention_scale_dk),
    "scale_sqrt_dc_plus_dr": ("attention", _attention_scale_dc),
    "key_and_value_swapped": ("decompress", lambda C, wk, wv: (C @ wv, C @ wk)),
    "value_from_key_projection": ("decompress", lambda C, wk, wv: (C @ wk, C @ wk)),
    "mask_excludes_current_token": ("visible_keys", lambda L, p, kr=None: np.arange(0, max(0, min(L, p)))),
    "mask_reads_one_future_token": ("visible_keys", lambda L, p, kr=None: np.arange(
        max(0, kr[0]) if kr else 0, max(max(0, kr[0]) if kr else 0, min(L, p + 2, kr[1] if kr else L)))),
    "lse_missing_max": ("softmax_lse", _softmax_lse_no_max),
    "merge_without_normalising": ("merge_partials", _merge_unnormalised),
    "gather_ignores_page_table": ("gather_rows", _gather_wrong),
    "rms_sum_instead_of_mean": ("rms_normalize", _rms_sum_not_mean),
    "rms_eps_outside_sqrt": ("rms_normalize", _rms_eps_outside_sqrt),
    "rms_multiplies_instead_of_divides": ("rms_normalize", _rms_multiplies),
    "rms_over_wrong_axis": ("rms_normalize", _rms_wrong_axis),
    "query_projections_swapped": ("query_parts", lambda h, dq, uq, qr: (
        np.asarray(h, F64) @ dq, np.einsum("...c,hck->...hk", np.asarray(h, F64) @ dq, np.asarray(qr, F64)),
        np.einsum("...c,hcr->...hr", np.asarray(h, F64) @ dq, np.asarray(uq, F64)))),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for name, pin in ALL_PINS.items():
        try:
            pin()
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            failed.append(f"{name}: {type(e).__name__}")
    assert failed, f"mutant {mutant} passed every pin"
