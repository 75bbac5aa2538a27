"""Plain fp64 exact attention: forward, blockwise-merge forward, backward.

TEST INFRASTRUCTURE (see the package docstring): slow, obviously correct, and
independent of the HIP library.

Layout of every tensor argument: [B, H, N, d] (d innermost), any float dtype;
values are upcast exactly to float64 before any arithmetic.  Results are
float64.  `lse` is [B, H, N], natural log.  K and V (and dK, dV) may carry
fewer heads, H_kv, than Q: grouped-query attention, or multi-query attention
when H_kv = 1 (everydayai.blog flash-attention article, "FlashAttention-2",
point 3, names both variants without defining them).  Reading used: H_kv
divides H and query head h reads key/value head h // (H / H_kv), so each run
of H / H_kv consecutive query heads shares one K/V head; dK and dV of a shared
head are the sums over its query heads (the chain rule through the sharing).

Definition followed (everydayai.blog flash-attention article, opening
``standard_attention`` snippet, and "The Math Behind Flash Attention",
formula 1): for each (b, h)

    s_ij     = scale * sum_k q_ik k_jk
    allowed  = (not causal or j <= i) and (no mask or mask[i//T][j//T] != 0)
    m_i      = max over allowed j of s_ij
    l_i      = sum over allowed j of exp(s_ij - m_i)
    P_ij     = exp(s_ij - m_i) / l_i   (allowed j),  0 otherwise
    O_i      = sum_j P_ij v_j
    lse_i    = m_i + ln l_i

A row with no allowed key gets O_i = 0 and lse_i = -inf (the pages never reach
that case; this is the reading used throughout).  The block-sparse mask follows
the FlashAttention abstract on Tri Dao's scite.ai page ("block-sparse
attention"): one uint8 [ceil(N/T), ceil(N/T)] tile mask shared by all (b, h),
nonzero = keep, ANDed with causality.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kv_head(h, n_heads, n_kv_heads):
    """Key/value head read by query head h (grouped-query reading in the header)."""
    if n_kv_heads < 1 or n_heads % n_kv_heads != 0:
        raise ValueError(f"{n_heads} query heads cannot share {n_kv_heads} key/value heads evenly")
    return h // (n_heads // n_kv_heads)


def allowed(rows, n_keys, causal, block_mask=None, mask_block=128, cols=None):
    """Boolean [len(rows), len(cols)]: True where key j is visible to query i."""
    r = np.asarray(rows, dtype=np.int64)[:, None]
    c = (np.arange(n_keys) if cols is None else np.asarray(cols, dtype=np.int64))[None, :]
    ok = np.ones((r.shape[0], c.shape[1]), dtype=bool)
    if causal:
        ok &= c <= r
    if block_mask is not None:
        bm = np.asarray(block_mask)
        ok &= bm[r // mask_block, c // mask_block] != 0
    return ok


def _visible_columns(rows, n_keys, causal, block_mask, mask_block):
    """Keys that at least one of `rows` may see; every other key has P = 0 exactly."""
    hi = int(np.max(rows)) + 1 if causal else n_keys
    if block_mask is None:
        return np.arange(hi)
    bm = np.asarray(block_mask)
    tiles = np.nonzero(np.any(bm[np.unique(np.asarray(rows) // mask_block)] != 0, axis=0))[0]
    cols = (tiles[:, None] * mask_block + np.arange(mask_block)[None, :]).ravel()
    return cols[cols < hi]


def _rows_one_head(q_rows, k, v, rows, scale, causal, block_mask, mask_block):
    """O and lse of the given query rows of one head, by the definition above."""
    cols = _visible_columns(rows, k.shape[0], causal, block_mask, mask_block)
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.full(len(rows), -np.inf)
    if cols.size == 0:
        return o, lse
    s = scale * (q_rows @ k[cols].T)
    ok = allowed(rows, k.shape[0], causal, block_mask, mask_block, cols=cols)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    m0 = np.where(has, m, 0.0)
    e = np.where(ok, np.exp(s - m0[:, None]), 0.0)
    l = e.sum(axis=1)
    o[has] = (e[has] @ v[cols]) / l[has, None]
    lse[has] = m0[has] + np.log(l[has])
    return o, lse


def forward_rows(q, k, v, rows, scale, causal=False, block_mask=None, mask_block=128):
    """O[:, :, rows] and lse[:, :, rows] of exact attention (rows shared by every head).

    Rows are evaluated one mask-row group at a time so that a block-sparse mask only
    touches the keys it keeps; the result is the definition above, unchanged.
    Returns (o [B, H, R, d], lse [B, H, R]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    B, H, N, d = q.shape
    o = np.zeros((B, H, rows.size, v.shape[-1]))
    lse = np.full((B, H, rows.size), -np.inf)
    if rows.size == 0:
        return o, lse
    if block_mask is None:
        groups = [np.arange(rows.size)]
    else:
        chunk = rows // mask_block
        groups = [np.nonzero(chunk == c)[0] for c in np.unique(chunk)]
    for b in range(B):
        for h in range(H):
            kh = kv_head(h, H, k.shape[1])
            for g in groups:
                o[b, h, g], lse[b, h, g] = _rows_one_head(
                    q[b, h, rows[g]], k[b, kh], v[b, kh], rows[g], scale, causal, block_mask, mask_block)
    return o, lse


def forward(q, k, v, scale, causal=False, block_mask=None, mask_block=128):
    """Every row of exact attention: (o [B, H, N, d], lse [B, H, N])."""
    N = np.shape(q)[2]
    return forward_rows(q, k, v, np.arange(N), scale, causal, block_mask, mask_block)


def _probs_one_head(q, k, ok, scale):
    s = np.where(ok, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    e = np.where(ok, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    p[has] = e[has] / l[has, None]
    return p


def probabilities(q, k, scale, causal=False, block_mask=None, mask_block=128):
    """The full attention matrix P [B, H, N, N] (small N only)."""
    q, k = _f64(q), _f64(k)
    B, H, N, _ = q.shape
    ok = allowed(np.arange(N), N, causal, block_mask, mask_block)
    p = np.zeros((B, H, N, N))
    for b in range(B):
        for h in range(H):
            p[b, h] = _probs_one_head(q[b, h], k[b, kv_head(h, H, k.shape[1])], ok, scale)
    return p


# ---------------------------------------------------------------------------
# Blockwise forward: the method itself, kept on the CPU so that it is pinned
# against the one-shot definition (everydayai.blog flash-attention article,
# "The Math Behind Flash Attention", formulas 1 and 2, and the blockwise loop
# under "Implementation Details").
#
# Reading of formula 2 (garbled as printed: it nests softmax inside softmax and
# carries no sums): for a row whose keys split into parts x and y with maxima
# m_x, m_y and sums l_x, l_y, the merged statistics are m = max(m_x, m_y) and
# l = e^(m_x - m) l_x + e^(m_y - m) l_y, and the merged output weights each
# part's *normalised* output by e^(m_part - m) l_part / l.  The printed
# blockwise loop rescales the old normalised output by e^(m_old - m_new) only,
# without the old sum; that is wrong as soon as a row spans two key blocks and
# is not followed here.
# ---------------------------------------------------------------------------

def merge_block(m_old, l_old, o_old, s_blk, v_blk):
    """Fold one key block into the running (m, l, normalised o) of a set of rows.

    s_blk: scaled scores [R, b] with -inf at masked keys; v_blk: [b, d].
    m_old = -inf means "no key seen yet"; its weight is then 0.
    """
    m_blk = s_blk.max(axis=1)
    m_new = np.maximum(m_old, m_blk)
    seen = np.isfinite(m_new)
    m0 = np.where(seen, m_new, 0.0)
    alpha = np.where(np.isfinite(m_old), np.exp(m_old - m0), 0.0)
    e = np.where(np.isfinite(s_blk), np.exp(s_blk - m0[:, None]), 0.0)
    l_new = alpha * l_old + e.sum(axis=1)
    num = (alpha * l_old)[:, None] * o_old + e @ v_blk
    o_new = np.zeros_like(o_old)
    o_new[seen] = num[seen] / l_new[seen, None]
    return m_new, l_new, o_new


def forward_blockwise(q, k, v, scale, causal=False, block_mask=None, mask_block=128, block=128):
    """Exact attention computed one key block at a time with the online merge.

    Must equal `forward` up to fp64 rounding for every block size >= 1.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    rows = np.arange(N)
    o_all = np.zeros((B, H, N, v.shape[-1]))
    lse_all = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            kh = kv_head(h, H, k.shape[1])
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            o = np.zeros((N, v.shape[-1]))
            for j0 in range(0, N, block):
                cols = np.arange(j0, min(j0 + block, N))
                ok = allowed(rows, N, causal, block_mask, mask_block, cols=cols)
                s = np.where(ok, scale * (q[b, h] @ k[b, kh, cols].T), -np.inf)
                m, l, o = merge_block(m, l, o, s, v[b, kh, cols])
            has = np.isfinite(m)
            o_all[b, h] = o
            lse_all[b, h, has] = m[has] + np.log(l[has])
    return o_all, lse_all


def merge_partials(lse_x, o_x, lse_y, o_y):
    """Combine two normalised partial results over disjoint key sets.

    lse = ln(e^lse_x + e^lse_y) and o = e^(lse_x - lse) o_x + e^(lse_y - lse) o_y,
    which is formula 2's reading above written with lse = m + ln l.
    """
    lse_x, lse_y = _f64(lse_x), _f64(lse_y)
    m = np.maximum(lse_x, lse_y)
    m0 = np.where(np.isfinite(m), m, 0.0)
    wx = np.where(np.isfinite(lse_x), np.exp(lse_x - m0), 0.0)
    wy = np.where(np.isfinite(lse_y), np.exp(lse_y - m0), 0.0)
    tot = wx + wy
    lse = np.where(tot > 0, m0 + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    safe = np.where(tot > 0, tot, 1.0)
    o = (wx / safe)[..., None] * _f64(o_x) + (wy / safe)[..., None] * _f64(o_y)
    return lse, o


# ---------------------------------------------------------------------------
# Backward.  The pages say only that the backward pass recomputes attention
# instead of storing it (everydayai.blog flash-attention article, "Enter Flash
# Attention", point 2).  The gradients are those of the forward definition for
# the loss L = sum(dO * O); recomputation does not change them.
#
#   dV = P^T dO          dP = dO V^T          D_i = sum_j P_ij dP_ij
#   dS = P * (dP - D)    dQ = scale dS K      dK = scale dS^T Q
# ---------------------------------------------------------------------------

def backward(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128, return_delta=False):
    """(dq [B, H, N, d], dk and dv [B, H_kv, N, d]) in float64; optionally also D [B, H, N]."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    N = q.shape[2]
    ok = allowed(np.arange(N), N, causal, block_mask, mask_block)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros(q.shape[:3])
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            kh = kv_head(h, H, k.shape[1])
            P = _probs_one_head(q[b, h], k[b, kh], ok, scale)
            dv[b, kh] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, kh].T
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            dq[b, h] = scale * (dS @ k[b, kh])
            dk[b, kh] += scale * (dS.T @ q[b, h])
            delta[b, h] = D
    if return_delta:
        return dq, dk, dv, delta
    return dq, dk, dv


def _row_groups(rows, block_mask, mask_block, chunk):
    """Consecutive pieces of the sorted `rows`: one mask row at a time when there is a block
    mask (so only the keys it keeps are touched), else `chunk` rows at a time."""
    if rows.size == 0:
        return []
    if block_mask is None:
        return [rows[i:i + chunk] for i in range(0, rows.size, chunk)]
    cut = np.nonzero(np.diff(rows // mask_block))[0] + 1
    return np.split(rows, cut)


def backward_rows(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128, rows=None, keys=None,
                  heads=None, chunk=512):
    """Part of the backward of `backward`, for checks at sizes where all of it is too slow.

    Returns (dq [B, H, R, d] of the query rows `rows`, dk and dv [B, H_kv, K, d] of the
    keys `keys`) in float64, with the same chain rule as `backward`:
    dV_j = sum_i P_ij dO_i, dK_j = scale sum_i dS_ij q_i, dQ_i = scale sum_j dS_ij k_j,
    dS_ij = P_ij (dP_ij - D_i), dP_ij = <dO_i, v_j>, D_i = <dO_i, O_i>.
    A key's gradient sums over every query that sees it, so the statistics (the row's
    softmax and D_i) are computed for all of those rows, not only the sampled ones.
    `heads`: optional list of the K/V heads (b, h_kv) to evaluate (all by default); the
    entries of the others stay zero, and dq is filled for their query heads only.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    hkv = k.shape[1]
    rows = np.unique(np.asarray([] if rows is None else rows, dtype=np.int64))
    keys = np.unique(np.asarray([] if keys is None else keys, dtype=np.int64))
    dq = np.zeros((B, H, rows.size, d))
    dk = np.zeros((B, hkv, keys.size, d))
    dv = np.zeros((B, hkv, keys.size, d))
    g = H // hkv
    todo = [(b, j) for b in range(B) for j in range(hkv)] if heads is None else list(heads)
    # rows that see at least one sampled key, plus the sampled rows themselves
    if keys.size:
        sees = allowed(np.arange(N), N, causal, block_mask, mask_block, cols=keys).any(axis=1)
    else:
        sees = np.zeros(N, dtype=bool)
    sees[rows] = True
    need = np.nonzero(sees)[0]
    row_pos = {int(r): i for i, r in enumerate(rows)}
    for b, kh in todo:
        K, V = k[b, kh], v[b, kh]
        for h in range(kh * g, (kh + 1) * g):
            if kv_head(h, H, hkv) != kh:
                raise AssertionError("query head outside its K/V group")
            for grp in _row_groups(need, block_mask, mask_block, chunk):
                cols = _visible_columns(grp, N, causal, block_mask, mask_block)
                if cols.size == 0:
                    continue
                Q, dO = q[b, h, grp], do[b, h, grp]
                ok = allowed(grp, N, causal, block_mask, mask_block, cols=cols)
                P = _probs_one_head(Q, K[cols], ok, scale)
                D = np.sum(dO * (P @ V[cols]), axis=1)
                # dQ of the sampled rows in this piece
                sel = np.array([i for i, r in enumerate(grp) if int(r) in row_pos], dtype=np.int64)
                if sel.size:
                    dS = P[sel] * (dO[sel] @ V[cols].T - D[sel, None])
                    dq[b, h, [row_pos[int(r)] for r in grp[sel]]] = scale * (dS @ K[cols])
                # dK, dV of the sampled keys this piece sees
                kin = np.nonzero(np.isin(keys, cols))[0]
                if kin.size:
                    at = np.searchsorted(cols, keys[kin])
                    Pk = P[:, at]
                    dSk = Pk * (dO @ V[keys[kin]].T - D[:, None])
                    dv[b, kh, kin] += Pk.T @ dO
                    dk[b, kh, kin] += scale * (dSk.T @ Q)
    return dq, dk, dv
