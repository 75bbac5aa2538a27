"""Planted mistakes in the oracle must be caught by its pins (the pins have teeth).

Each mutation replaces one internal step of `oracle.attention` with a plausible
wrong version (a dropped term, a wrong sign or index, a transposed operand) and
requires that at least one pin fails.  Everything runs on the CPU.
"""

import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention as oatt

_orig_rows = oatt._rows_one_head
_orig_allowed = oatt.allowed
_orig_probs = oatt._probs_one_head


def _rows_no_max_shift_in_lse(q_rows, k, v, rows, scale, causal, bm, mb):
    o, lse = _orig_rows(q_rows, k, v, rows, scale, causal, bm, mb)
    cols = oatt._visible_columns(rows, k.shape[0], causal, bm, mb)
    if cols.size == 0:
        return o, lse
    s = np.where(oatt.allowed(rows, k.shape[0], causal, bm, mb, cols=cols), scale * (q_rows @ k[cols].T), -np.inf)
    m = s.max(axis=1)
    return o, np.where(np.isfinite(m), lse - m, lse)  # lse without the row maximum


def _rows_transposed_k(q_rows, k, v, rows, scale, causal, bm, mb):
    n = min(k.shape[0], k.shape[1])
    k2 = k.copy()
    k2[:n, :n] = k[:n, :n].T
    return _orig_rows(q_rows, k2, v, rows, scale, causal, bm, mb)


def _rows_no_scale(q_rows, k, v, rows, scale, causal, bm, mb):
    return _orig_rows(q_rows, k, v, rows, 1.0, causal, bm, mb)


def _rows_v_off_by_one(q_rows, k, v, rows, scale, causal, bm, mb):
    return _orig_rows(q_rows, k, np.roll(v, 1, axis=0), rows, scale, causal, bm, mb)


def _allowed_strict_causal(rows, n_keys, causal, block_mask=None, mask_block=128, cols=None):
    ok = _orig_allowed(rows, n_keys, False, block_mask, mask_block, cols)
    if causal:
        r = np.asarray(rows)[:, None]
        c = (np.arange(n_keys) if cols is None else np.asarray(cols))[None, :]
        ok &= c < r  # j < i instead of j <= i
    return ok


def _allowed_mask_transposed(rows, n_keys, causal, block_mask=None, mask_block=128, cols=None):
    bm = None if block_mask is None else np.asarray(block_mask).T
    return _orig_allowed(rows, n_keys, causal, bm, mask_block, cols)


def _merge_block_drop_old_l(m_old, l_old, o_old, s_blk, v_blk):
    """The printed blockwise loop's update: the old normalised output is not re-weighted by the old sum."""
    m_blk = s_blk.max(axis=1)
    m_new = np.maximum(m_old, m_blk)
    seen = np.isfinite(m_new)
    m0 = np.where(seen, m_new, 0.0)
    alpha = np.where(np.isfinite(m_old), np.exp(m_old - m0), 0.0)
    e = np.where(np.isfinite(s_blk), np.exp(s_blk - m0[:, None]), 0.0)
    l_new = alpha * l_old + e.sum(axis=1)
    num = alpha[:, None] * o_old + e @ v_blk
    o_new = np.zeros_like(o_old)
    o_new[seen] = num[seen] / l_new[seen, None]
    return m_new, l_new, o_new


def _probs_row_sum_off(q, k, ok, scale):
    p = _orig_probs(q, k, ok, scale)
    return p * 1.001


def _backward_sign_flip(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128, return_delta=False):
    out = list(_orig_backward(q, k, v, do, scale, causal, block_mask, mask_block, True))
    out[1] = -out[1]  # dK with the wrong sign
    return tuple(out) if return_delta else tuple(out[:3])


def _backward_delta_dropped(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128, return_delta=False):
    q64, k64, v64, do64 = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    N = q64.shape[2]
    ok = oatt.allowed(np.arange(N), N, causal, block_mask, mask_block)
    dq, dk, dv = np.zeros_like(q64), np.zeros_like(k64), np.zeros_like(v64)
    D = np.zeros(q64.shape[:3])
    for b in range(q64.shape[0]):
        for h in range(q64.shape[1]):
            kh = oatt.kv_head(h, q64.shape[1], k64.shape[1])
            P = oatt._probs_one_head(q64[b, h], k64[b, kh], ok, scale)
            dv[b, kh] += P.T @ do64[b, h]
            dS = P * (do64[b, h] @ v64[b, kh].T)  # the "- D" term dropped
            dq[b, h] = scale * dS @ k64[b, kh]
            dk[b, kh] += scale * dS.T @ q64[b, h]
    return (dq, dk, dv, D) if return_delta else (dq, dk, dv)


def _kv_head_interleaved(h, n_heads, n_kv_heads):
    return h % n_kv_heads  # query heads dealt round-robin instead of in consecutive runs


def _backward_group_not_summed(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128,
                               return_delta=False):
    """dK/dV of a shared K/V head taken from the last query head of its group only (assigned, not added)."""
    B, H, N, d = np.shape(q)
    hkv = np.shape(k)[1]
    g = H // hkv
    out = list(_orig_backward(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), do, scale, causal,
                              block_mask, mask_block, True))
    out[1] = out[1].reshape(B, hkv, g, N, d)[:, :, -1]
    out[2] = out[2].reshape(B, hkv, g, N, d)[:, :, -1]
    return tuple(out) if return_delta else tuple(out[:3])


_orig_backward = oatt.backward
_orig_backward_rows = oatt.backward_rows


def _backward_rows_sampled_queries_only(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128,
                                        rows=None, keys=None, heads=None, chunk=512):
    """dK/dV of the sampled keys summed over the sampled query rows only (not every row that sees
    them): dO zeroed outside the sampled rows, which leaves their dQ as it was."""
    rows = np.unique(np.asarray([] if rows is None else rows, dtype=np.int64))
    keep = np.zeros(np.shape(q)[2], dtype=bool)
    keep[rows] = True
    do = np.where(keep[None, None, :, None], np.asarray(do, dtype=np.float64), 0.0)
    return _orig_backward_rows(q, k, v, do, scale, causal, block_mask, mask_block, rows, keys, heads, chunk)


MUTATIONS = {
    "lse_without_max": ("_rows_one_head", _rows_no_max_shift_in_lse, pins.FORWARD_CHECKS),
    "k_transposed": ("_rows_one_head", _rows_transposed_k, pins.FORWARD_CHECKS),
    "scale_dropped": ("_rows_one_head", _rows_no_scale, pins.FORWARD_CHECKS),
    "v_index_shifted": ("_rows_one_head", _rows_v_off_by_one, pins.FORWARD_CHECKS),
    "causal_strict": ("allowed", _allowed_strict_causal, pins.FORWARD_CHECKS),
    "block_mask_transposed": ("allowed", _allowed_mask_transposed, pins.FORWARD_CHECKS),
    "merge_drops_old_l": ("merge_block", _merge_block_drop_old_l, [pins.check_blockwise_equals_one_shot]),
    "probs_not_normalised": ("_probs_one_head", _probs_row_sum_off, pins.ALL_CHECKS),
    "dk_sign": ("backward", _backward_sign_flip, pins.BACKWARD_CHECKS),
    "delta_dropped": ("backward", _backward_delta_dropped, pins.BACKWARD_CHECKS),
    "kv_heads_interleaved": ("kv_head", _kv_head_interleaved, pins.ALL_CHECKS),
    "gqa_grads_not_summed": ("backward", _backward_group_not_summed, pins.BACKWARD_CHECKS),
    "sampled_keys_see_sampled_rows_only": ("backward_rows", _backward_rows_sampled_queries_only,
                                           [pins.check_backward_rows]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn, checks = MUTATIONS[name]
    monkeypatch.setattr(oatt, attr, fn)
    import oracle

    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    bad = pins.failing_checks(checks)
    assert bad, f"mutation {name} passed every pin"


# --------------------------------------------------------------------------- FP8 part
import oracle_pins_fp8 as pins8  # noqa: E402
from oracle import fp8 as of8  # noqa: E402

_orig_fwht = of8.fwht_fp32
_orig_scale_exponent = of8.scale_exponent
_orig_bound = of8.pv_rounding_bound


def _e4m3_round_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a >= 2.0 ** -6, a, 1.0)))
    step = np.where(a >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9)
    return np.copysign(np.floor(a / step + 0.5) * step, x)  # halves away from zero


def _scale_exponent_one_high(amax):
    return _orig_scale_exponent(amax) + (1 if amax else 0)


def _fwht_difference_flipped(x, signs):
    y = np.array(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = b - a  # wrong sign
        h *= 2
    return y


def _fwht_signs_ignored(x, signs):
    return _orig_fwht(x, np.ones(np.shape(x)[-1]))


def _bound_not_normalised(q, k, v, scale, causal=False, rows=None):
    """The bound without the division by the row sum l."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    N = q.shape[2]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    b = _orig_bound(q, k, v, scale, causal, rows)
    s = scale * np.einsum("bhnd,bhmd->bhnm", q[:, :, rows], np.repeat(k, q.shape[1] // k.shape[1], axis=1))
    if causal:
        s = np.where(np.arange(N)[None, :] <= rows[:, None], s, -np.inf)
    l = np.exp(s - s.max(axis=-1, keepdims=True)).sum(axis=-1)
    return b * l[..., None]


FP8_MUTATIONS = {
    "e4m3_ties_away_from_zero": ("e4m3_round", _e4m3_round_ties_away),
    "scale_exponent_one_high": ("scale_exponent", _scale_exponent_one_high),
    "fwht_difference_flipped": ("fwht_fp32", _fwht_difference_flipped),
    "rotation_signs_ignored": ("fwht_fp32", _fwht_signs_ignored),
    "bound_not_normalised": ("pv_rounding_bound", _bound_not_normalised),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_planted_fp8_mistake_is_caught(name, monkeypatch):
    attr, fn = FP8_MUTATIONS[name]
    monkeypatch.setattr(of8, attr, fn)
    bad = []
    for c in pins8.FP8_CHECKS:
        try:
            with np.errstate(all="ignore"):
                c()
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            bad.append(c.__name__)
    assert bad, f"mutation {name} passed every FP8 pin"


# --------------------------------------------------------------------------- bf16 backward bound
from oracle import bounds as obnd  # noqa: E402

_orig_u = obnd.U_BF16


@pytest.mark.parametrize("name,attr,value", [
    ("bf16_unit_roundoff_halved", "U_BF16", _orig_u / 2.0),   # the fraction-bit count off by one
    ("bf16_unit_roundoff_doubled", "U_BF16", _orig_u * 2.0),  # loose enough to be near-vacuous
])
def test_planted_bound_mistake_is_caught(name, attr, value, monkeypatch):
    monkeypatch.setattr(obnd, attr, value)
    try:
        pins.check_bf16_backward_bound()
    except AssertionError:
        return
    raise AssertionError(f"mutation {name} passed the bf16 bound pin")
