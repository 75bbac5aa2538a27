"""Brute-force attention in pure Python -- TEST INFRASTRUCTURE for tiny inputs.

This is the plain definition (everydayai.blog flash-attention article, opening
``standard_attention`` snippet: scores, softmax over keys, weighted sum of V)
evaluated literally, with no maximum subtraction: each weight is exp(s_ij) and
the normaliser is their exactly rounded sum (math.fsum).  It therefore shares
neither code nor arithmetic order with `oracle.attention`, which uses the
max-shifted form of formula 1 in "The Math Behind Flash Attention".  Keep the
inputs small (|s| well below 700) so that exp does not overflow.
"""

from __future__ import annotations

import math

import numpy as np


def _visible(i, j, causal, block_mask, mask_block):
    if causal and j > i:
        return False
    if block_mask is not None and block_mask[i // mask_block][j // mask_block] == 0:
        return False
    return True


def brute_forward(q, k, v, scale, causal=False, block_mask=None, mask_block=128):
    """(o, lse) as nested float64 numpy arrays, computed element by element."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, N, dv))
    lse = np.full((B, H, N), -math.inf)
    bm = None if block_mask is None else np.asarray(block_mask).tolist()
    Hkv = k.shape[1]
    for b in range(B):
        for h in range(H):
            # grouped-query sharing: query head h reads key/value head floor(h * H_kv / H)
            Q = q[b, h].tolist()
            K = k[b, h * Hkv // H].tolist()
            V = v[b, h * Hkv // H].tolist()
            for i in range(N):
                w = {}
                for j in range(N):
                    if _visible(i, j, causal, bm, mask_block):
                        s = scale * math.fsum(Q[i][t] * K[j][t] for t in range(d))
                        w[j] = math.exp(s)
                if not w:
                    continue
                z = math.fsum(w.values())
                for c in range(dv):
                    o[b, h, i, c] = math.fsum(w[j] * V[j][c] for j in w) / z
                lse[b, h, i] = math.log(z)
    return o, lse


def brute_backward_fd(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128, rel_step=1e-6):
    """Central finite differences of L = sum(dO * O) with respect to q, k and v.

    Uses `brute_forward` for O, so it depends on no gradient formula.
    Cost: 6 * B*H*N*d forward evaluations -- tiny shapes only.
    """
    q = np.array(q, dtype=np.float64)
    k = np.array(k, dtype=np.float64)
    v = np.array(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)

    def loss():
        o, _ = brute_forward(q, k, v, scale, causal, block_mask, mask_block)
        return math.fsum((o * do).ravel().tolist())

    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        flat = x.reshape(-1)
        gflat = g.reshape(-1)
        for idx in range(flat.size):
            x0 = flat[idx]
            h = rel_step * max(1.0, abs(x0))
            flat[idx] = x0 + h
            lp = loss()
            flat[idx] = x0 - h
            lm = loss()
            flat[idx] = x0
            gflat[idx] = (lp - lm) / (2.0 * h)
        grads.append(g)
    return tuple(grads)
