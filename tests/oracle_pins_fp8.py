"""Pins of the FP8 part of the oracle (oracle/fp8.py); each check raises AssertionError when it is wrong.

What fixes the expected values, independently of the oracle's code: torch's own
float8_e4m3fn conversions (a library routine, round to nearest even), scipy's
Hadamard matrix, the orthogonality of the rotation, exact integer arithmetic,
and a step-by-step simulation of the kernel's rounding of P for the error bound.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import attention as oatt
from oracle import fp8 as of8


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([35, 900, seed]))


def _torch_codes(x32):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def check_e4m3_vs_torch(seed=0):
    """Decoding of all 256 codes, and rounding/encoding of values across every binade, the
    subnormals and exact ties, equal torch's float8_e4m3fn conversions."""
    import torch

    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = of8.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin]) and np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    rng = _rng(seed)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-14, 6, 20000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    grid = np.unique(np.abs(got[fin]))
    ties = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)  # exact midpoints: ties to even
    x = np.concatenate([x, ties, -ties, grid.astype(np.float32), np.float32([0.0, -0.0, 448.0, 463.9])])
    assert np.array_equal(of8.e4m3_encode(x), _torch_codes(x))
    assert np.array_equal(of8.e4m3_round(x), of8.e4m3_decode(_torch_codes(x)))


def check_fwht_vs_hadamard(seed=1):
    """The fp32 transform equals x diag(sigma) H_d with scipy's Hadamard matrix, exactly on
    integer inputs (every partial sum is an exact fp32 integer), and applying it twice gives d x."""
    from scipy.linalg import hadamard

    rng = _rng(seed)
    for d in (2, 4, 8, 16, 32, 64, 128):
        Hd = hadamard(d).astype(np.float64)
        assert np.array_equal(of8.fwht_fp32(np.eye(d, dtype=np.float32), np.ones(d)), Hd)
        x = rng.integers(-1000, 1000, size=(3, 5, d)).astype(np.float32)
        s = rng.choice([-1.0, 1.0], size=d)
        y = of8.fwht_fp32(x, s)
        assert np.array_equal(y, (x.astype(np.float64) * s) @ Hd)
        assert np.array_equal(of8.fwht_fp32(y, np.ones(d)), d * x.astype(np.float64) * s)
        xf = rng.standard_normal((4, d)).astype(np.float32)
        yf = of8.fwht_fp32(xf, s)
        assert np.max(np.abs(yf - (xf.astype(np.float64) * s) @ Hd)) <= 1e-5 * max(1.0, np.abs(yf).max())


def check_scale_exponent(seed=2):
    """The block exponent is the smallest integer e with amax 2^-e <= 448, for amax around every
    power of two and at the exact boundaries 448 * 2^k."""
    rng = _rng(seed)
    vals = list(np.exp2(rng.uniform(-60, 60, 2000)))
    for k in range(-20, 21):
        b = 448.0 * 2.0 ** k
        vals += [b, np.nextafter(b, 0.0), np.nextafter(b, np.inf), 2.0 ** k]
    for a in vals:
        e = of8.scale_exponent(a)
        assert a * 2.0 ** -e <= 448.0 and a * 2.0 ** -(e - 1) > 448.0, a
    assert of8.scale_exponent(0.0) == 0


def check_quantize(seed=3):
    """Codes equal torch's conversion of the block-scaled (rotated) values; the exponent is
    minimal (the block maximum lands in [224, 448]); scales are 2^e (times fl32(1/sqrt(d)) when
    rotated); zero blocks stay zero; dequantised values are within half a code step."""
    rng = _rng(seed)
    for d in (64, 128):
        x = (rng.standard_normal((2, 3, 300, d)) * np.exp(rng.uniform(-3, 3, (2, 3, 300, 1)))).astype(np.float32)
        x[0, 1, :128] = 0.0                  # an all-zero block
        x[1, 2, 5, 7] = 3000.0               # an outlier
        x = x.astype(np.float32)
        for signs in (None, rng.choice([-1.0, 1.0], size=d)):
            codes, scales = of8.quantize(x, signs)
            y = of8.fwht_fp32(x, signs) if signs is not None else x
            r = np.float32(1.0 / math.sqrt(d)) if signs is not None else np.float32(1.0)
            assert scales.shape == (2, 3, 3) and codes.shape == x.shape
            for b in range(2):
                for h in range(3):
                    for i in range(3):
                        rows = slice(128 * i, min(300, 128 * (i + 1)))
                        e = math.frexp(float(scales[b, h, i] / r))[1] - 1
                        assert scales[b, h, i] == np.float32(np.ldexp(r, e))
                        yb = y[b, h, rows]
                        ref = _torch_codes(np.ldexp(yb, -e).astype(np.float32))
                        assert np.array_equal(codes[b, h, rows], ref)
                        dec = of8.e4m3_decode(codes[b, h, rows])
                        if np.all(yb == 0):
                            assert e == 0 and np.all(dec == 0)
                            continue
                        assert 224.0 <= np.max(np.abs(dec)) <= 448.0
                        a = np.abs(np.ldexp(yb.astype(np.float64), -e))
                        tol = np.where(a >= 2.0 ** -6, a * 2.0 ** -4, 2.0 ** -10)
                        assert np.all(np.abs(dec - np.ldexp(yb.astype(np.float64), -e)) <= tol)


def check_rotation_preserves_scores(seed=4):
    """(Q M)(K M)^T = Q K^T for M = diag(sigma) H_d / sqrt(d) (M orthogonal), so the rotated,
    quantised Q and K give the scores of the originals within the quantisation error."""
    from scipy.linalg import hadamard

    rng = _rng(seed)
    for d in (64, 128):
        s = rng.choice([-1.0, 1.0], size=d)
        M = np.diag(s) @ hadamard(d) / math.sqrt(d)
        assert np.max(np.abs(M @ M.T - np.eye(d))) <= 1e-14
        q = rng.standard_normal((1, 2, 200, d)).astype(np.float32)
        k = rng.standard_normal((1, 2, 200, d)).astype(np.float32)
        exact = q.astype(np.float64) @ np.swapaxes(k.astype(np.float64), -1, -2)
        rot = (q.astype(np.float64) @ M) @ np.swapaxes(k.astype(np.float64) @ M, -1, -2)
        assert np.max(np.abs(rot - exact)) <= 1e-11
        dq = of8.dequantize(*of8.quantize(q, s))
        dk = of8.dequantize(*of8.quantize(k, s))
        approx = dq @ np.swapaxes(dk, -1, -2)
        # each coordinate carries a relative rounding error of at most 2^-4 (normal range)
        bound = 2.0 ** -3 * (np.abs(dq) @ np.swapaxes(np.abs(dk), -1, -2)) + 1e-3
        assert np.all(np.abs(approx - exact) <= bound)
        assert np.sqrt(np.mean((approx - exact) ** 2)) <= 0.05 * np.sqrt(np.mean(exact ** 2))


def check_incoherent_processing_helps(seed=5):
    """With a few outlier coordinates in Q and K, attention of the rotated, quantised inputs is
    closer to exact attention of the originals than attention of the unrotated, quantised ones."""
    rng = _rng(seed)
    d, N = 64, 256
    q = rng.standard_normal((1, 2, N, d))
    k = rng.standard_normal((1, 2, N, d))
    v = rng.standard_normal((1, 2, N, d))
    q[..., :2] *= 60.0
    k[..., :2] *= 60.0
    q, k, v = (a.astype(np.float32) for a in (q, k, v))
    scale = 1.0 / math.sqrt(d) / 8.0
    ref, _ = oatt.forward(q, k, v, scale, True)
    s = rng.choice([-1.0, 1.0], size=d)
    v8 = of8.quantize(v)
    plain, _ = of8.forward_fp8(*of8.quantize(q), *of8.quantize(k), *v8, scale, True)
    rot, _ = of8.forward_fp8(*of8.quantize(q, s), *of8.quantize(k, s), *v8, scale, True)
    e_plain = np.sqrt(np.mean((plain - ref) ** 2))
    e_rot = np.sqrt(np.mean((rot - ref) ** 2))
    assert e_rot < 0.8 * e_plain, (e_rot, e_plain)


def _simulate_kernel_rounding(q, k, v, scale, causal, tile=64):
    """O of a key-tile loop with a running row maximum that rounds P to e4m3 before P.V
    (sums of P unrounded) -- the arithmetic the bound is about, in float64."""
    B, H, N, d = q.shape
    out = np.zeros((B, H, N, d))
    for b in range(B):
        for h in range(H):
            kh = oatt.kv_head(h, H, k.shape[1])
            s_all = scale * (q[b, h] @ k[b, kh].T)
            if causal:
                s_all = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], s_all, -np.inf)
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for j0 in range(0, N, tile):
                st = s_all[:, j0:j0 + tile]
                mn = np.maximum(m, st.max(axis=1))
                alpha = np.where(np.isfinite(m), np.exp(m - mn), 0.0)
                p = np.where(np.isfinite(st), np.exp(st - mn[:, None]), 0.0)
                acc = acc * alpha[:, None] + of8.e4m3_round(p) @ v[b, kh, j0:j0 + tile]
                l = l * alpha + p.sum(axis=1)
                m = mn
            out[b, h] = acc / l[:, None]
    return out


def check_pv_rounding_bound(seed=6):
    """The bound holds for a simulation of the kernel's rounding of P (running maximum per
    64-key tile), on diffuse and on peaked score rows, and is not vacuous."""
    rng = _rng(seed)
    worst = 0.0
    for mult, causal in ((1.0, False), (1.0, True), (3.0, True), (0.2, False)):
        q = rng.standard_normal((1, 2, 300, 64)) * mult
        k = rng.standard_normal((1, 1, 300, 64)) * mult
        v = rng.standard_normal((1, 1, 300, 64))
        scale = 0.125
        ref, _ = oatt.forward(q, k, v, scale, causal)
        sim = _simulate_kernel_rounding(q, k, v, scale, causal)
        bound = of8.pv_rounding_bound(q, k, v, scale, causal)
        err = np.abs(sim - ref)
        assert np.all(err <= bound * (1 + 1e-9) + 1e-14), float(np.max(err - bound))
        worst = max(worst, float(np.max(err / bound)))
        # not vacuous: the typical element's error is within a factor of a few hundred of it
        assert np.median(err / bound) > 2e-3, float(np.median(err / bound))
    assert worst > 0.1, worst


FP8_CHECKS = [
    check_e4m3_vs_torch,
    check_fwht_vs_hadamard,
    check_scale_exponent,
    check_quantize,
    check_rotation_preserves_scores,
    check_incoherent_processing_helps,
    check_pv_rounding_bound,
]
