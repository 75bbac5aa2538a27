"""FP8 (e4m3) quantisation with incoherent processing, and the FP8 forward -- TEST INFRASTRUCTURE.

Slow and plain; shares no code with the HIP library.  Source: the everydayai.blog
flash-attention article, section "FlashAttention-3": FP8 support (low-precision
arithmetic for speed) and incoherent processing (a technique that reduces the
quantisation error of low-precision formats).  The pages define neither, so the
readings below are the ones used (each is listed in the design notes):

* FP8 is OCP E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals 2^-9 * m, largest finite value 448, no infinities (the fp8 format
  of the MI355X matrix cores).  Values are rounded to nearest, ties to even.
* Quantisation is per block of 128 consecutive rows of one (b, h): with y the
  (possibly rotated) rows, the block's scale exponent e is the smallest integer
  with max|y| * 2^-e <= 448, the code of y is RNE_e4m3(y * 2^-e), and the stored
  scale is 2^e * r, with r = fl32(1/sqrt(d)) for rotated blocks and 1 otherwise,
  so that code * scale approximates the rotated row.  A block of zeros gets e = 0.
* Incoherent processing multiplies Q and K (never V) by one random orthogonal
  matrix M = diag(sigma) H_d / sqrt(d), sigma a vector of random signs and H_d
  the Sylvester Hadamard matrix ([[H, H], [H, -H]]).  (Q M)(K M)^T = Q K^T: the
  scores do not change, but a few large coordinates are spread over all d of
  them before rounding.  y = x diag(sigma) H_d is computed in fp32 by the fast
  Walsh-Hadamard transform, stages h = 1, 2, 4, ..., d/2 in that order, each
  replacing (a, b) = (y_i, y_{i+h}) for every i with bit h clear by (a + b, a - b);
  1/sqrt(d) goes into the scale.  fp32 and this stage order are the precision
  in which the codes are decided, so both sides reproduce them bit for bit.
* The FP8 forward is exact attention of the dequantised Q, K, V (`forward_fp8`);
  the kernel additionally rounds P to e4m3 before P.V, with P taken relative to a
  basis at or below the running row maximum (so P >= its value relative to the
  final maximum, and P stays far below 448).  `pv_rounding_bound` bounds what that
  rounding can change for any such basis.

Parity status: e4m3 rounding, encoding and decoding are pinned against torch's
float8_e4m3fn conversions; the transform against scipy's Hadamard matrix (exactly,
on integer inputs) and orthogonality; quantisation against torch's conversion of
the scaled values and the minimality of the exponent; the bound against a
simulation of the rounding (tests/test_oracle_fp8.py).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _f64, forward, kv_head

E4M3_MAX = 448.0
SCALE_BLOCK = 128  # rows per quantisation scale
_MIN_NORMAL = 2.0 ** -6
_SUB_STEP = 2.0 ** -9


def e4m3_round(x):
    """Nearest e4m3 value of each element (ties to even), as float64; |x| must not exceed 464."""
    x = _f64(x)
    a = np.abs(x)
    if np.any(a >= 464.0) or not np.all(np.isfinite(x)):
        raise ValueError("value outside the finite e4m3 range")
    # spacing of the grid at |x|: 2^-9 below 2^-6, else 2^(floor(log2|x|) - 3)
    e = np.floor(np.log2(np.where(a >= _MIN_NORMAL, a, 1.0)))
    step = np.where(a >= _MIN_NORMAL, np.exp2(e - 3), _SUB_STEP)
    q = np.round(a / step) * step  # np.round rounds halves to even; a / step is exact
    return np.copysign(q, x)


def e4m3_encode(x):
    """uint8 codes of the e4m3-rounded values of x (sign bit 7, exponent bits 6..3, mantissa 2..0)."""
    q = e4m3_round(x)
    a = np.abs(q)
    sign = np.signbit(q).astype(np.uint8) << 7
    normal = a >= _MIN_NORMAL
    e = np.floor(np.log2(np.where(normal, a, 1.0))).astype(np.int64)
    mant_n = np.where(normal, a / np.exp2(e) * 8.0 - 8.0, 0.0)
    code_n = ((e + 7) << 3) + mant_n.astype(np.int64)
    code_s = (a / _SUB_STEP).astype(np.int64)
    return (sign | np.where(normal, code_n, code_s).astype(np.uint8)).astype(np.uint8)


def e4m3_decode(codes):
    """float64 values of uint8 e4m3 codes (0x7F and 0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m * _SUB_STEP, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def fwht_fp32(x, signs):
    """x diag(signs) H_d along the last axis in fp32, stage by stage (h = 1, 2, ..., d/2)."""
    y = np.array(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b  # fp32 + fp32, rounded once
        v[..., 1, :] = a - b
        h *= 2
    return y


def scale_exponent(amax):
    """Smallest integer e with amax * 2^-e <= 448 (0 when amax == 0), exactly."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    mant, ex = math.frexp(amax)  # amax = mant * 2^ex, mant in [0.5, 1)
    # 448 = 0.875 * 2^9: amax <= 448 * 2^e  <=>  mant * 2^(ex - 9 - e) <= 0.875
    return ex - 9 if mant <= 0.875 else ex - 8


def quantize(x, signs=None, block=SCALE_BLOCK):
    """(codes uint8 [B, H, N, d], scales float32 [B, H, ceil(N / block)]) of x [B, H, N, d].

    signs (d values of +-1) turns on incoherent processing (the rotation above).
    """
    x32 = np.asarray(x, dtype=np.float32)
    B, H, N, d = x32.shape
    y = fwht_fp32(x32, signs) if signs is not None else x32.copy()
    r = np.float32(1.0 / math.sqrt(d)) if signs is not None else np.float32(1.0)
    nb = -(-N // block)
    codes = np.zeros((B, H, N, d), dtype=np.uint8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                rows = slice(i * block, min(N, (i + 1) * block))
                yb = y[b, h, rows]
                e = scale_exponent(np.max(np.abs(yb)))
                codes[b, h, rows] = e4m3_encode(np.ldexp(yb.astype(np.float64), -e))
                scales[b, h, i] = np.ldexp(r, e)
    return codes, scales


def dequantize(codes, scales, block=SCALE_BLOCK):
    """float64 values code * scale of a quantised [B, H, N, d] tensor."""
    vals = e4m3_decode(codes)
    N = vals.shape[2]
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :N]
    return vals * s[..., None]


def forward_fp8(q8, qs, k8, ks, v8, vs, scale, causal=False):
    """Exact attention of the dequantised inputs: (o [B, H, N, d], lse [B, H, N]) in float64.

    K and V may have H_kv heads (grouped-query, as in `oracle.attention`).
    """
    return forward(dequantize(q8, qs), dequantize(k8, ks), dequantize(v8, vs), scale, causal)


def pv_rounding_bound(q, k, v, scale, causal=False, rows=None):
    """Per-element bound of |O_kernel - O| caused by rounding P to e4m3, for float64 inputs.

    With P_ij = exp(s_ij - m_i) (m_i the row maximum, so P <= 1; a kernel basis at
    or below it only makes its P larger, by the factor its result is later scaled
    down with), rounding P to e4m3 moves it
    by at most 2^-4 P for P >= 2^-6 and by at most 2^-10 below; O_i divides by
    l_i = sum_j P_ij, which the kernel sums from the unrounded P.  Hence
      |dO_ic| <= (2^-4 sum_{P_ij >= 2^-6} P_ij |v_jc| + 2^-10 sum_{P_ij < 2^-6} |v_jc|) / l_i.
    Returns [B, H, R, d] for the query rows `rows` (all rows by default).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, H, rows.size, v.shape[-1]))
    cols = np.arange(N)[None, :]
    ok = np.ones((rows.size, N), dtype=bool) if not causal else cols <= rows[:, None]
    for b in range(B):
        for h in range(H):
            kh = kv_head(h, H, k.shape[1])
            s = np.where(ok, scale * (q[b, h, rows] @ k[b, kh].T), -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.where(ok, np.exp(s - m), 0.0)
            l = p.sum(axis=1, keepdims=True)
            big = p >= _MIN_NORMAL
            av = np.abs(v[b, kh])
            out[b, h] = (2.0 ** -4 * (np.where(big, p, 0.0) @ av) + 2.0 ** -10 * ((ok & ~big) @ av)) / l
    return out
