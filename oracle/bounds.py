"""Rounding-error bound of a bf16 attention backward -- TEST INFRASTRUCTURE.

Slow and plain; shares no code with the HIP library.  The pages fix no precision
for the GPU path; the one bounded here is bf16 inputs with fp32 arithmetic and
three bf16 roundings (the reading used for the bf16 path, listed in the design
notes):

  * forward: P = exp(s - m) in fp32, rounded to bf16 for the P.V product; the
    row sum l from the unrounded P; the output O = (P V) / l stored in bf16;
  * backward: D_i = <dO_i, O_i> from that stored O; P recomputed in fp32 from
    the saved lse; dP = dO V^T in fp32; dS = P (dP - D) rounded to bf16 for
    dQ = scale dS K and dK = scale dS^T Q; P rounded to bf16 for dV = P^T dO.

With u = 2^-8 (bf16 keeps 8 significant bits; round to nearest), the scores'
fp32 sums bounded in the worst case (d 2^-24 of the sum of the products'
magnitudes, which moves P relatively by that much, and the row's lse likewise),
and f = 2^-16 standing for every other fp32 evaluation (exp2, products and
sums, relative to the magnitudes they act on; fp32's own unit is 2^-24), each element's error is bounded, to first order, by propagating
absolute values through those steps (`bf16_backward_bound`).  The bound is a
worst case (every rounding in the same direction); actual errors sit well below
it.  Pinned in tests/oracle_pins.py against a step-by-step simulation of the
roundings (check_bf16_backward_bound).
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, _probs_one_head, allowed, kv_head

U_BF16 = 2.0 ** -8
F_FP32 = 2.0 ** -16


def bf16_backward_bound(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128, row_block=2048):
    """Per-element bounds (dq [B, H, N, d], dk and dv [B, H_kv, N, d]) of |g_kernel - g|.

    Rows are taken `row_block` at a time (the bound of dK and dV sums over rows), so
    that the N x N intermediates stay small at long N.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    u, f = U_BF16, F_FP32
    sc = abs(scale)
    B, H, N, d = q.shape
    bq = np.zeros_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            kh = kv_head(h, H, k.shape[1])
            K, V = k[b, kh], v[b, kh]
            aK, aV = np.abs(K), np.abs(V)
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                Q, dO = q[b, h, rows], do[b, h, rows]
                ok = allowed(rows, N, causal, block_mask, mask_block)
                P = _probs_one_head(Q, K, ok, scale)
                O = P @ V
                dP = dO @ V.T
                D = np.sum(dO * O, axis=1)
                dS = P * (dP - D[:, None])
                adO = np.abs(dO)
                # relative error of P evaluated in fp32: the score sums (d products each, worst
                # case d 2^-24 of the sum of their magnitudes), the same for the row's lse, and f
                es = (d * 2.0 ** -24) * sc * (np.abs(Q) @ aK.T)
                eP = np.where(ok, es + np.max(np.where(ok, es, 0.0), axis=1, keepdims=True) + f, 0.0)
                # stored output: P rounded for P.V, then O rounded to bf16
                eO = (P * (u + eP)) @ aV + (u + f) * np.abs(O)
                # D from the stored output, summed in fp32
                eD = np.sum(adO * eO, axis=1) + f * np.sum(adO * np.abs(O), axis=1)
                # dS before its rounding: D's error, P's error and the fp32 subtraction
                e1 = P * (eD[:, None] + (eP + f) * (np.abs(dP) + np.abs(D)[:, None]))
                # after rounding to bf16, plus the fp32 sums of the two products
                e2 = e1 + u * (np.abs(dS) + e1) + f * (np.abs(dS) + e1)
                bq[b, h, rows] = sc * (e2 @ aK)
                bk[b, kh] += sc * (e2.T @ np.abs(Q))
                bv[b, kh] += (P * (u + eP + 2.0 * f)).T @ adO
    return bq, bk, bv
