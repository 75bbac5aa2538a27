"""Pins of the fp64 oracle: each check raises AssertionError when the oracle is wrong.

The checks are plain functions so that the mutation tests can run them against
an oracle with a planted mistake and require that at least one of them fails.
Each states what fixes the expected value independently of the oracle's code.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from oracle import attention as oatt

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(seed, shape, mult=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape) * mult


def _eval(x):
    """Golden files write closed forms such as "log(3)"; evaluate with math only."""
    if isinstance(x, list):
        return [_eval(e) for e in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"log": math.log, "sqrt": math.sqrt, "exp": math.exp}))
    return float(x)


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    arr = {}
    for key in ("q", "k", "v", "do"):
        if key in g:
            arr[key] = np.asarray(_eval(g[key]))[None, None]
    return g, arr


# --------------------------------------------------------------------------- forward

def check_brute_force(seed=0):
    """Oracle == literal definition (no max shift, fsum) on tiny inputs, every mask kind."""
    cases = []
    for N in (1, 2, 3, 4, 7, 16, 17):
        for d in (1, 2, 3, 8):
            for causal in (False, True):
                cases.append((N, d, causal, None))
    for N, mb in ((7, 2), (16, 4), (17, 4)):
        nb = -(-N // mb)
        rng = np.random.default_rng(seed + N)
        mask = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
        np.fill_diagonal(mask, 1)
        for causal in (False, True):
            cases.append((N, 3, causal, (mask, mb)))
        mask0 = mask.copy()
        mask0[0, :] = 0  # rows of tile 0 see nothing: fully masked rows
        cases.append((N, 3, False, (mask0, mb)))
    for i, (N, d, causal, m) in enumerate(cases):
        B, H = (1, 2) if N < 8 else (1, 1)
        q = _rand(seed * 1000 + 3 * i, (B, H, N, d))
        k = _rand(seed * 1000 + 3 * i + 1, (B, H, N, d))
        v = _rand(seed * 1000 + 3 * i + 2, (B, H, N, d + 1))
        scale = 1.0 / math.sqrt(d)
        bm, mb = (None, 128) if m is None else m
        o, lse = oracle.forward(q, k, v, scale, causal, bm, mb)
        ob, lseb = oracle.brute_forward(q, k, v, scale, causal, bm, mb)
        assert np.max(np.abs(o - ob)) <= 1e-12, (N, d, causal, np.max(np.abs(o - ob)))
        fin = np.isfinite(lseb)
        assert np.array_equal(fin, np.isfinite(lse)), (N, d, causal)
        assert np.max(np.abs(lse[fin] - lseb[fin]), initial=0.0) <= 1e-12, (N, d, causal)


def check_rows_sum_to_one(seed=1):
    """Rows of P sum to 1 (softmax decomposition, formula 1)."""
    for causal in (False, True):
        q = _rand(seed, (2, 2, 33, 8), 2.0)
        k = _rand(seed + 1, (2, 2, 33, 8), 2.0)
        p = oracle.probabilities(q, k, 0.5, causal)
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-13
        if causal:
            assert np.all(np.triu(np.ones((33, 33)), 1)[None, None] * p == 0)


def check_constant_v(seed=2):
    """v_j = c for all j gives O_i = c; a column of ones in V gives a column of ones in O."""
    for causal in (False, True):
        for bm in (None, np.array([[1, 0, 1], [0, 1, 1], [1, 1, 1]], dtype=np.uint8)):
            q = _rand(seed, (1, 2, 40, 5), 3.0)
            k = _rand(seed + 1, (1, 2, 40, 5), 3.0)
            c = np.array([2.5, -1.0, 0.0, 7.0])
            v = np.broadcast_to(c, (1, 2, 40, 4)).copy()
            o, _ = oracle.forward(q, k, v, 0.7, causal, bm, 16)
            assert np.max(np.abs(o - c)) <= 1e-13 * 7.0
            v2 = _rand(seed + 2, (1, 2, 40, 4))
            v2[..., 1] = 1.0
            o2, _ = oracle.forward(q, k, v2, 0.7, causal, bm, 16)
            assert np.max(np.abs(o2[..., 1] - 1.0)) <= 1e-13


def check_special_cases(seed=3):
    """Closed forms: N=1, Q=0 (and scale=0), causal row 0, two keys = logistic, scale sign."""
    v = _rand(seed, (1, 1, 1, 6))
    q = _rand(seed + 1, (1, 1, 1, 6))
    k = _rand(seed + 2, (1, 1, 1, 6))
    o, lse = oracle.forward(q, k, v, 0.3, False)
    assert np.max(np.abs(o - v)) == 0.0
    assert abs(lse[0, 0, 0] - 0.3 * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14
    N = 9
    v = _rand(seed + 3, (1, 1, N, 4))
    k = _rand(seed + 4, (1, 1, N, 4))
    for q, scale in ((np.zeros((1, 1, N, 4)), 0.5), (_rand(seed + 5, (1, 1, N, 4)), 0.0)):
        o, lse = oracle.forward(q, k, v, scale, False)
        assert np.max(np.abs(o - v.mean(axis=2, keepdims=True))) <= 1e-13
        assert np.max(np.abs(lse - math.log(N))) <= 1e-13
        o, lse = oracle.forward(q, k, v, scale, True)
        csum = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        assert np.max(np.abs(o - csum)) <= 1e-13
        assert np.max(np.abs(lse[0, 0] - np.log(np.arange(1, N + 1)))) <= 1e-13
    q = _rand(seed + 6, (1, 1, N, 4))
    o, lse = oracle.forward(q, k, v, 0.5, True)
    assert np.max(np.abs(o[0, 0, 0] - v[0, 0, 0])) == 0.0
    # two keys: P_i0 = logistic(s_i0 - s_i1)
    q = _rand(seed + 7, (1, 1, 2, 3), 2.0)
    k = _rand(seed + 8, (1, 1, 2, 3), 2.0)
    v = _rand(seed + 9, (1, 1, 2, 3))
    o, lse = oracle.forward(q, k, v, 0.8, False)
    for i in range(2):
        s0 = 0.8 * float(np.dot(q[0, 0, i], k[0, 0, 0]))
        s1 = 0.8 * float(np.dot(q[0, 0, i], k[0, 0, 1]))
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert np.max(np.abs(o[0, 0, i] - (p0 * v[0, 0, 0] + (1 - p0) * v[0, 0, 1]))) <= 1e-13
        assert abs(lse[0, 0, i] - (s0 + math.log1p(math.exp(s1 - s0)))) <= 1e-13
    # a negative scale is the positive scale applied to -Q
    q = _rand(seed + 10, (1, 2, 11, 4))
    k = _rand(seed + 11, (1, 2, 11, 4))
    v = _rand(seed + 12, (1, 2, 11, 4))
    for causal in (False, True):
        a = oracle.forward(q, k, v, -0.6, causal)
        b = oracle.forward(-q, k, v, 0.6, causal)
        assert np.max(np.abs(a[0] - b[0])) <= 1e-14 and np.max(np.abs(a[1] - b[1])) <= 1e-14


def check_diagonal_mask_is_chunked_causal(seed=4):
    """A diagonal-only tile mask with causal == independent causal attention on each tile-row chunk."""
    N, mb = 20, 8
    nb = -(-N // mb)
    q = _rand(seed, (1, 2, N, 3), 2.0)
    k = _rand(seed + 1, (1, 2, N, 3), 2.0)
    v = _rand(seed + 2, (1, 2, N, 3))
    o, lse = oracle.forward(q, k, v, 0.6, True, np.eye(nb, dtype=np.uint8), mb)
    for c0 in range(0, N, mb):
        sl = slice(c0, min(c0 + mb, N))
        oc, lc = oracle.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.6, True)
        assert np.max(np.abs(o[:, :, sl] - oc)) <= 1e-13
        assert np.max(np.abs(lse[:, :, sl] - lc)) <= 1e-13


def check_mask_equivalences(seed=5):
    """All-ones tile mask == dense; lower-triangular all-ones mask + causal == causal dense."""
    N, mb = 37, 8
    nb = -(-N // mb)
    q = _rand(seed, (2, 1, N, 4), 2.0)
    k = _rand(seed + 1, (2, 1, N, 4), 2.0)
    v = _rand(seed + 2, (2, 1, N, 4))
    for causal in (False, True):
        a = oracle.forward(q, k, v, 0.5, causal)
        b = oracle.forward(q, k, v, 0.5, causal, np.ones((nb, nb), np.uint8), mb)
        assert np.max(np.abs(a[0] - b[0])) <= 1e-13 and np.max(np.abs(a[1] - b[1])) <= 1e-13
    a = oracle.forward(q, k, v, 0.5, True)
    b = oracle.forward(q, k, v, 0.5, True, np.tril(np.ones((nb, nb), np.uint8)), mb)
    assert np.max(np.abs(a[0] - b[0])) <= 1e-13 and np.max(np.abs(a[1] - b[1])) <= 1e-13


def check_rows_subset(seed=6):
    """Sampled-row evaluation equals the same rows of the full evaluation."""
    N, mb = 45, 8
    nb = -(-N // mb)
    q = _rand(seed, (1, 2, N, 4), 2.0)
    k = _rand(seed + 1, (1, 2, N, 4), 2.0)
    v = _rand(seed + 2, (1, 2, N, 4))
    rows = np.array([0, 1, 7, 8, 22, 44])
    mask = np.tril((np.random.default_rng(seed).random((nb, nb)) < 0.5).astype(np.uint8))
    np.fill_diagonal(mask, 1)
    for causal, bm in ((False, None), (True, None), (True, mask)):
        of, lf = oracle.forward(q, k, v, 0.5, causal, bm, mb)
        orow, lrow = oracle.forward_rows(q, k, v, rows, 0.5, causal, bm, mb)
        assert np.max(np.abs(of[:, :, rows] - orow)) <= 1e-13
        assert np.max(np.abs(lf[:, :, rows] - lrow)) <= 1e-13


def check_blockwise_equals_one_shot(seed=7):
    """The online merge over key blocks reproduces the one-shot softmax (formula 2's purpose)."""
    N = 50
    q = _rand(seed, (1, 2, N, 4), 3.0)
    k = _rand(seed + 1, (1, 2, N, 4), 3.0)
    v = _rand(seed + 2, (1, 2, N, 4))
    mask = np.tril((np.random.default_rng(seed).random((7, 7)) < 0.5).astype(np.uint8))
    np.fill_diagonal(mask, 1)
    for causal, bm in ((False, None), (True, None), (True, mask)):
        ref = oracle.forward(q, k, v, 0.9, causal, bm, 8)
        for block in (1, 3, 16, 128, N):
            got = oracle.forward_blockwise(q, k, v, 0.9, causal, bm, 8, block)
            assert np.max(np.abs(got[0] - ref[0])) <= 1e-12, (causal, block)
            assert np.max(np.abs(got[1] - ref[1])) <= 1e-12, (causal, block)


def check_merge_partials(seed=8):
    """Merging the results over two disjoint key sets equals attention over their union."""
    N = 30
    q = _rand(seed, (1, 1, N, 4), 3.0)
    k = _rand(seed + 1, (1, 1, N, 4), 3.0)
    v = _rand(seed + 2, (1, 1, N, 4))
    perm = np.random.default_rng(seed).permutation(N)
    x, y = perm[:11], perm[11:]
    ox, lx = oracle.forward(q, k[:, :, x], v[:, :, x], 0.7, False)
    oy, ly = oracle.forward(q, k[:, :, y], v[:, :, y], 0.7, False)
    lse, o = oracle.merge_partials(lx, ox, ly, oy)
    of, lf = oracle.forward(q, k, v, 0.7, False)
    assert np.max(np.abs(o - of)) <= 1e-13 and np.max(np.abs(lse - lf)) <= 1e-13


def check_torch_sdpa(seed=9):
    """Oracle == torch's own fp64 CPU scaled_dot_product_attention and logsumexp (a library routine)."""
    import torch

    for causal, use_mask in ((False, False), (True, False), (False, True), (True, True)):
        N, mb = 27, 4
        nb = -(-N // mb)
        q = _rand(seed, (2, 3, N, 5), 2.0)
        k = _rand(seed + 1, (2, 3, N, 5), 2.0)
        v = _rand(seed + 2, (2, 3, N, 5))
        bm = None
        vis = np.ones((N, N), dtype=bool)
        if causal:
            vis &= np.tril(np.ones((N, N), dtype=bool))
        if use_mask:
            bm = (np.random.default_rng(seed).random((nb, nb)) < 0.6).astype(np.uint8)
            np.fill_diagonal(bm, 1)
            vis &= np.kron(bm, np.ones((mb, mb), dtype=np.uint8))[:N, :N].astype(bool)
        tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
        tm = torch.from_numpy(vis)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=0.45)
        s = (tq @ tk.transpose(-1, -2)) * 0.45
        lse_ref = torch.logsumexp(s.masked_fill(~tm, float("-inf")), dim=-1)
        o, lse = oracle.forward(q, k, v, 0.45, causal, bm, mb)
        assert np.max(np.abs(o - ref.numpy())) <= 1e-12
        assert np.max(np.abs(lse - lse_ref.numpy())) <= 1e-12


def check_golden_forward():
    """Hand-derived closed forms (tests/golden)."""
    g, a = load_golden("two_keys_logistic.json")
    for mode, causal in (("noncausal", False), ("causal", True)):
        o, lse = oracle.forward(a["q"], a["k"], a["v"], g["scale"], causal)
        assert np.max(np.abs(o[0, 0] - np.asarray(_eval(g[mode]["o"])))) <= 1e-13
        assert np.max(np.abs(lse[0, 0] - np.asarray(_eval(g[mode]["lse"])))) <= 1e-13
    g, a = load_golden("zero_query_block_mask.json")
    bm = np.asarray(g["block_mask"], dtype=np.uint8)
    for mode, causal in (("noncausal", False), ("causal", True)):
        o, lse = oracle.forward(a["q"], a["k"], a["v"], g["scale"], causal, bm, g["mask_block"])
        assert np.max(np.abs(o[0, 0] - np.asarray(_eval(g[mode]["o"])))) <= 1e-13
        assert np.max(np.abs(lse[0, 0] - np.asarray(_eval(g[mode]["lse"])))) <= 1e-13


def check_gqa_forward(seed=13):
    """Grouped-/multi-query forward == torch fp64 SDPA with enable_gqa, == brute force, == K/V heads repeated."""
    import torch

    for hkv in (1, 2, 3, 6):
        for causal in (False, True):
            q = _rand(seed, (2, 6, 21, 5), 2.0)
            k = _rand(seed + 1, (2, hkv, 21, 5), 2.0)
            v = _rand(seed + 2, (2, hkv, 21, 5))
            o, lse = oracle.forward(q, k, v, 0.45, causal)
            tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, is_causal=causal, scale=0.45, enable_gqa=True)
            assert np.max(np.abs(o - ref.numpy())) <= 1e-12, (hkv, causal)
            # each K/V head repeated for its run of consecutive query heads: plain multi-head attention
            rk, rv = np.repeat(k, 6 // hkv, axis=1), np.repeat(v, 6 // hkv, axis=1)
            o2, lse2 = oracle.forward(q, rk, rv, 0.45, causal)
            assert np.max(np.abs(o - o2)) <= 1e-13 and np.max(np.abs(lse - lse2)) <= 1e-13
    q, k, v = _rand(seed + 3, (1, 4, 6, 3)), _rand(seed + 4, (1, 2, 6, 3)), _rand(seed + 5, (1, 2, 6, 3))
    bm = np.array([[1, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    for causal, mask in ((False, None), (True, None), (True, bm)):
        o, lse = oracle.forward(q, k, v, 0.8, causal, mask, 2)
        ob, lseb = oracle.brute_forward(q, k, v, 0.8, causal, mask, 2)
        assert np.max(np.abs(o - ob)) <= 1e-13 and np.max(np.abs(lse - lseb)) <= 1e-13


FORWARD_CHECKS = [
    check_brute_force,
    check_rows_sum_to_one,
    check_constant_v,
    check_special_cases,
    check_diagonal_mask_is_chunked_causal,
    check_mask_equivalences,
    check_rows_subset,
    check_blockwise_equals_one_shot,
    check_merge_partials,
    check_torch_sdpa,
    check_golden_forward,
    check_gqa_forward,
]


# --------------------------------------------------------------------------- backward

def check_finite_differences(seed=10):
    """Gradients == central finite differences of sum(dO * O) through the brute-force forward."""
    shapes = [(1, 1, 1, 2), (1, 1, 2, 1), (1, 1, 3, 2), (1, 2, 5, 3), (1, 1, 8, 4)]
    for i, shp in enumerate(shapes):
        for causal in (False, True):
            q = _rand(seed + 4 * i, shp)
            k = _rand(seed + 4 * i + 1, shp)
            v = _rand(seed + 4 * i + 2, shp)
            do = _rand(seed + 4 * i + 3, shp)
            scale = 0.7
            got = oracle.backward(q, k, v, do, scale, causal)
            fd = oracle.brute_backward_fd(q, k, v, do, scale, causal)
            for g, f in zip(got, fd):
                err = np.max(np.abs(g - f)) / max(1.0, np.max(np.abs(f)))
                assert err <= 1e-6, (shp, causal, err)
    # a block mask with mask_block=2 on N=6, plus a fully masked tile row
    bm = np.array([[0, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    q, k, v, do = (_rand(seed + 50 + t, (1, 1, 6, 2)) for t in range(4))
    got = oracle.backward(q, k, v, do, 0.9, True, bm, 2)
    fd = oracle.brute_backward_fd(q, k, v, do, 0.9, True, bm, 2)
    for g, f in zip(got, fd):
        assert np.max(np.abs(g - f)) / max(1.0, np.max(np.abs(f))) <= 1e-6


def check_torch_autograd(seed=11):
    """Gradients == torch fp64 autograd through scaled_dot_product_attention."""
    import torch

    for causal in (False, True):
        q, k, v, do = (_rand(seed + t, (2, 2, 19, 6)) for t in range(4))
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.4)
        (out * torch.from_numpy(do)).sum().backward()
        got = oracle.backward(q, k, v, do, 0.4, causal)
        for g, t in zip(got, (tq.grad, tk.grad, tv.grad)):
            assert np.max(np.abs(g - t.numpy())) <= 1e-12


def check_backward_invariants(seed=12):
    """sum_j dK_j = 0; sum_j dV_j = sum_i dO_i; <Q,dQ> = <K,dK>; Q=0 closed forms; D = rowsum(dO*O)."""
    for causal in (False, True):
        q, k, v, do = (_rand(seed + t, (1, 2, 23, 5), 2.0) for t in range(4))
        dq, dk, dv, D = oracle.backward(q, k, v, do, 0.5, causal, return_delta=True)
        nrm = max(1.0, np.abs(dk).max())
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12 * nrm
        assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= 1e-12 * max(1.0, np.abs(dv).max())
        lhs = np.sum(q * dq, axis=(2, 3))
        rhs = np.sum(k * dk, axis=(2, 3))
        assert np.max(np.abs(lhs - rhs)) <= 1e-11 * max(1.0, np.abs(lhs).max())
        o, _ = oracle.forward(q, k, v, 0.5, causal)
        assert np.max(np.abs(D - np.sum(do * o, axis=-1))) <= 1e-12
    k, v, do = (_rand(seed + 10 + t, (1, 1, 17, 3)) for t in range(3))
    dq, dk, dv = oracle.backward(np.zeros((1, 1, 17, 3)), k, v, do, 0.5, False)
    assert np.max(np.abs(dk)) <= 1e-14
    assert np.max(np.abs(dv - do.mean(axis=2, keepdims=True))) <= 1e-14


def check_golden_backward():
    """Hand-derived gradients of the two-key case (tests/golden)."""
    g, a = load_golden("two_keys_logistic.json")
    for mode, causal in (("noncausal", False), ("causal", True)):
        dq, dk, dv = oracle.backward(a["q"], a["k"], a["v"], a["do"], g["scale"], causal)
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert np.max(np.abs(got[0, 0] - np.asarray(_eval(g[mode][name])))) <= 1e-13, (mode, name)


def check_gqa_backward(seed=14):
    """Grouped-/multi-query gradients == central finite differences, == torch fp64 autograd with enable_gqa.

    dK and dV of a shared head must be the sums over its query heads: with K/V
    heads repeated per query head (plain multi-head attention), the group sums of
    the per-head gradients.
    """
    import torch

    for hkv, shp in ((1, (1, 3, 4, 2)), (2, (1, 4, 5, 2))):
        for causal in (False, True):
            q = _rand(seed, shp)
            k = _rand(seed + 1, (shp[0], hkv) + shp[2:])
            v = _rand(seed + 2, (shp[0], hkv) + shp[2:])
            do = _rand(seed + 3, shp)
            got = oracle.backward(q, k, v, do, 0.7, causal)
            fd = oracle.brute_backward_fd(q, k, v, do, 0.7, causal)
            for g, f in zip(got, fd):
                assert g.shape == f.shape
                assert np.max(np.abs(g - f)) / max(1.0, np.max(np.abs(f))) <= 1e-6, (hkv, causal)
    for hkv in (1, 2, 4):
        for causal in (False, True):
            q, do = _rand(seed + 10, (2, 4, 19, 6)), _rand(seed + 11, (2, 4, 19, 6))
            k, v = _rand(seed + 12, (2, hkv, 19, 6)), _rand(seed + 13, (2, hkv, 19, 6))
            tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
            out = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, is_causal=causal, scale=0.4, enable_gqa=True)
            (out * torch.from_numpy(do)).sum().backward()
            got = oracle.backward(q, k, v, do, 0.4, causal)
            for g, t in zip(got, (tq.grad, tk.grad, tv.grad)):
                assert np.max(np.abs(g - t.numpy())) <= 1e-12, (hkv, causal)
            g = 4 // hkv
            rq = oracle.backward(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), do, 0.4, causal)
            assert np.max(np.abs(got[0] - rq[0])) <= 1e-13
            for a, r in ((got[1], rq[1]), (got[2], rq[2])):
                assert np.max(np.abs(a - r.reshape(2, hkv, g, 19, 6).sum(axis=2))) <= 1e-12


def check_backward_rows(seed=17):
    """The sampled backward (dQ of some rows, dK/dV of some keys) equals the full backward at
    those rows and keys -- dense and causal, with a block mask (tile 4), with grouped heads,
    ragged lengths, empty row or key sets -- and equals torch fp64 autograd on a grouped case."""
    import torch

    cases = ((1, 2, 2, 23, 3, False, False), (2, 4, 2, 30, 4, True, False), (1, 3, 1, 29, 2, True, True),
             (2, 2, 2, 17, 5, False, True), (1, 4, 4, 1, 3, True, False))
    for i, (B, H, hkv, N, d, causal, masked) in enumerate(cases):
        q, do = _rand(seed + 10 * i, (B, H, N, d)), _rand(seed + 10 * i + 1, (B, H, N, d))
        k, v = _rand(seed + 10 * i + 2, (B, hkv, N, d)), _rand(seed + 10 * i + 3, (B, hkv, N, d))
        mb = 4
        mask = None
        if masked:
            nb = -(-N // mb)
            mask = (np.random.default_rng(seed + i).random((nb, nb)) < 0.5).astype(np.uint8)
            mask[nb // 2, :] = 0  # a mask row with no visible key
        full = oracle.backward(q, k, v, do, 0.6, causal, block_mask=mask, mask_block=mb)
        rng = np.random.default_rng(seed + 100 + i)
        for rows, keys in ((rng.choice(N, min(N, 7), replace=False), rng.choice(N, min(N, 6), replace=False)),
                           ([], np.arange(N)), (np.arange(N), [])):
            got = oracle.backward_rows(q, k, v, do, 0.6, causal, block_mask=mask, mask_block=mb, rows=rows,
                                       keys=keys, chunk=5)
            r, c = np.unique(np.asarray(rows, dtype=np.int64)), np.unique(np.asarray(keys, dtype=np.int64))
            assert np.max(np.abs(got[0] - full[0][:, :, r]), initial=0.0) <= 1e-12, (i, "dq")
            assert np.max(np.abs(got[1] - full[1][:, :, c]), initial=0.0) <= 1e-12, (i, "dk")
            assert np.max(np.abs(got[2] - full[2][:, :, c]), initial=0.0) <= 1e-12, (i, "dv")
    q, do = _rand(seed + 90, (1, 4, 26, 5)), _rand(seed + 91, (1, 4, 26, 5))
    k, v = _rand(seed + 92, (1, 2, 26, 5)), _rand(seed + 93, (1, 2, 26, 5))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.45, enable_gqa=True)
    (out * torch.from_numpy(do)).sum().backward()
    rows, keys = [0, 3, 11, 25], [0, 1, 12, 25]
    got = oracle.backward_rows(q, k, v, do, 0.45, True, rows=rows, keys=keys, heads=[(0, 1)])
    assert np.max(np.abs(got[0][:, 2:] - tq.grad.numpy()[:, 2:, rows])) <= 1e-12
    assert np.max(np.abs(got[0][:, :2])) == 0.0  # query heads of K/V head 0 were not asked for
    assert np.max(np.abs(got[1][:, 1] - tk.grad.numpy()[:, 1, keys])) <= 1e-12
    assert np.max(np.abs(got[2][:, 1] - tv.grad.numpy()[:, 1, keys])) <= 1e-12


def _bf16(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def _simulate_bf16_backward(q, k, v, do, scale, causal):
    """A bf16 kernel's arithmetic, step by step: fp32 evaluation, P rounded to bf16 for P.V
    and P^T dO, O stored in bf16 and used for D, dS rounded to bf16 for dQ and dK."""
    f32 = np.float32
    B, H, N, d = q.shape
    out = [np.zeros((B, H, N, d)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            kh = oatt.kv_head(h, H, k.shape[1])
            Q, K, V, dO = (a.astype(f32) for a in (q[b, h], k[b, kh], v[b, kh], do[b, h]))
            s = (f32(scale) * (Q @ K.T)).astype(f32)
            if causal:
                s = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], s, f32(-np.inf))
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m).astype(f32)
            l = p.sum(axis=1, keepdims=True, dtype=f32)
            O = _bf16((_bf16(p).astype(f32) @ V) / l).astype(f32)        # stored forward output
            lse = (m + np.log(l)).astype(f32)
            P = np.exp(s - lse).astype(f32)                               # recomputed from lse
            D = np.sum(dO * O, axis=1, keepdims=True, dtype=f32)
            dS = _bf16(P * ((dO @ V.T).astype(f32) - D)).astype(f32)
            out[0][b, h] = f32(scale) * (dS @ K)
            out[1][b, h] = f32(scale) * (dS.T @ Q)
            out[2][b, h] = _bf16(P).astype(f32).T @ dO
    return out


def check_bf16_backward_bound(seed=16):
    """The bf16 rounding bound holds for a step-by-step simulation of the roundings it is
    about, on diffuse and peaked rows, causal or not, and is not vacuous."""
    worst = 0.0
    for mult, causal in ((1.0, False), (1.7, True), (3.0, True), (0.3, False)):
        q, k, v, do = (_rand(seed + t, (1, 2, 96, 16), mult if t < 2 else 1.0) for t in range(4))
        q, k, v, do = (_bf16(a) for a in (q, k, v, do))
        scale = 0.25
        ref = oracle.backward(q, k, v, do, scale, causal)
        sim = _simulate_bf16_backward(q, k, v, do, scale, causal)
        bnd = oracle.bf16_backward_bound(q, k, v, do, scale, causal)
        for g, r, e in zip(sim, ref, bnd):
            err = np.abs(g - r)
            assert np.all(err <= e), float(np.max(err - e))
            worst = max(worst, float(np.max(err / e)))
            assert np.median(err / e) > 1e-3, float(np.median(err / e))
    assert worst > 0.5, worst  # the bound is reached within a factor of 2


BACKWARD_CHECKS = [
    check_backward_rows,
    check_bf16_backward_bound,
    check_finite_differences,
    check_torch_autograd,
    check_backward_invariants,
    check_golden_backward,
    check_gqa_backward,
]

ALL_CHECKS = FORWARD_CHECKS + BACKWARD_CHECKS


def failing_checks(checks=ALL_CHECKS):
    """Names of the checks that fail (used with a mutated oracle)."""
    bad = []
    for c in checks:
        try:
            with np.errstate(all="ignore"):
                c()
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            bad.append(c.__name__)
    return bad


__all__ = ["FORWARD_CHECKS", "BACKWARD_CHECKS", "ALL_CHECKS", "failing_checks", "oatt"]
