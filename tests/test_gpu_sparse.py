"""GPU block-sparse forward parity against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_35_amd import api, inputs
from gpu_util import bf16_store_ratio, TOL_BF16, TOL_LSE, announce, dev, host, max_err, report

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def run_sparse(q, k, v, mask, scale, causal):
    o, lse = api.forward_blocksparse(dev(q, BF), dev(k, BF), dev(v, BF),
                                     torch.from_numpy(np.ascontiguousarray(mask)).to("cuda:0"), scale, causal)
    torch.cuda.synchronize()
    return host(o), host(lse)


def test_blocksparse_64k_workload_sampled_rows():
    w = inputs.WORKLOADS["blocksparse_s64k"]
    announce(w.name)
    q, k, v, _ = inputs.make_qkv(w)
    nb = w.N // inputs.MASK_BLOCK
    mask = inputs.make_block_mask(nb, w.density, w.index, causal=w.causal)
    o, lse = run_sparse(q, k, v, mask, w.scale, w.causal)
    rows = inputs.sample_rows(w.N, w.sample_rows, w.index)
    ro, rl = oracle.forward_rows(q, k, v, rows, w.scale, w.causal, mask, inputs.MASK_BLOCK)
    eo, el = max_err(o[:, :, rows], ro), max_err(lse[:, :, rows], rl)
    report(w.name, o=eo, lse=el, rows=float(rows.size))
    assert eo <= TOL_BF16 and el <= TOL_LSE
    assert np.all(np.isfinite(o))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_random_masks(d, causal):
    for n in (1, 100, 128, 129, 500, 1030):
        nb = -(-n // 128)
        announce(f"sparse N={n} d={d} causal={causal}")
        q, k, v, _ = inputs.random_case(21, 1, 2, n, d, "bf16", mult=1.5)
        mask = inputs.random_block_mask(n, nb, 0.4, causal)
        if nb > 2:
            mask[1, :] = 0  # a tile row with no visible key: O = 0, lse = -inf
        if nb > 3:
            mask[2, :] = 0  # the first of a workgroup's two mask rows empty, the second not
        scale = api.default_scale(d)
        o, lse = run_sparse(q, k, v, mask, scale, causal)
        ro, rl = oracle.forward(q, k, v, scale, causal, mask, inputs.MASK_BLOCK)
        eo, el = max_err(o, ro), max_err(lse, rl)
        report(f"sparse N={n} d={d} causal={causal}", o=eo, lse=el)
        assert eo <= TOL_BF16 and el <= TOL_LSE, (n, d, causal)


@pytest.mark.parametrize("d", [64, 128])
def test_full_masks_equal_dense(d):
    """All-ones mask == dense; lower-triangular all-ones mask + causal == causal dense.

    The block-sparse kernel walks smaller key tiles than the dense one, so the two
    agree to rounding (each is checked against the oracle), not bit for bit.
    """
    n = 700
    nb = -(-n // 128)
    announce(f"sparse == dense d={d}")
    q, k, v, _ = inputs.random_case(22, 2, 2, n, d, "bf16")
    for causal, mask in ((False, np.ones((nb, nb), np.uint8)), (True, np.ones((nb, nb), np.uint8)),
                         (True, np.tril(np.ones((nb, nb), np.uint8)))):
        os_, ls_ = run_sparse(q, k, v, mask, 0.1, causal)
        o, lse = api.forward(dev(q, BF), dev(k, BF), dev(v, BF), 0.1, causal)
        torch.cuda.synchronize()
        ro, rl = oracle.forward(q, k, v, 0.1, causal)
        for oo, ll in ((os_, ls_), (host(o), host(lse))):
            assert max_err(oo, ro) <= TOL_BF16 and max_err(ll, rl) <= TOL_LSE, (d, causal)
        assert max_err(os_, host(o)) <= TOL_BF16 and max_err(ls_, host(lse)) <= TOL_LSE, (d, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_backward(d, causal):
    """fa_bwd_blocksparse against the oracle's gradients of the masked attention."""
    for n in (100, 129, 500, 1030):
        nb = -(-n // 128)
        announce(f"sparse bwd N={n} d={d} causal={causal}")
        # N(0, 1) activations as in the workloads: with sharper logits the bf16 rounding of
        # P and dS alone approaches the 2e-2 bound (as it does for the dense backward)
        q, k, v, do = inputs.random_case(23, 1, 2, n, d, "bf16", backward=True)
        mask = inputs.random_block_mask(24, nb, 0.4, causal)
        if nb > 2:
            mask[1, :] = 0  # a mask row with no visible key: its dQ is 0
        if nb > 3:
            mask[:, 2] = 0  # a mask column no query sees: its dK, dV are 0
        scale = api.default_scale(d)
        tm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda:0")
        tq, tk, tv, tdo = dev(q, BF), dev(k, BF), dev(v, BF), dev(do, BF)
        o, lse = api.forward_blocksparse(tq, tk, tv, tm, scale, causal)
        dq, dk, dv = api.backward(tq, tk, tv, o, lse, tdo, scale, causal, block_mask=tm)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.backward(q, k, v, do, scale, causal, mask, inputs.MASK_BLOCK)
        eq, ek, ev = max_err(host(dq), rq), max_err(host(dk), rk), max_err(host(dv), rv)
        report(f"sparse bwd N={n} d={d} causal={causal}", dq=eq, dk=ek, dv=ev)
        assert eq <= TOL_BF16 and ek <= TOL_BF16 and ev <= TOL_BF16, (n, d, causal)


@pytest.mark.parametrize("d", [64, 128])
def test_blocksparse_backward_full_mask_equals_dense(d):
    n = 600
    nb = -(-n // 128)
    announce(f"sparse bwd == dense d={d}")
    q, k, v, do = inputs.random_case(25, 1, 2, n, d, "bf16", backward=True)
    tq, tk, tv, tdo = dev(q, BF), dev(k, BF), dev(v, BF), dev(do, BF)
    for causal in (False, True):
        tm = torch.ones((nb, nb), dtype=torch.uint8, device="cuda:0")
        o, lse = api.forward(tq, tk, tv, 0.1, causal)
        sparse = api.backward(tq, tk, tv, o, lse, tdo, 0.1, causal, block_mask=tm)
        dense = api.backward(tq, tk, tv, o, lse, tdo, 0.1, causal)
        torch.cuda.synchronize()
        for a_, b_ in zip(sparse, dense):
            assert max_err(host(a_), host(b_)) <= TOL_BF16, (d, causal)


def test_blocksparse_backward_many_windows_bf16_gradients():
    """N = 4500 (18 query blocks of 256: two full windows of paired mask rows and a partial
    one), a random causal mask with an empty row and column, bf16 gradient outputs (their
    rounding adds up to 2^-8 of each value, hence twice the bf16 gate)."""
    n, d = 4500, 64
    nb = -(-n // 128)
    announce(f"sparse bwd N={n} d={d} bf16 gradients")
    q, k, v, do = inputs.random_case(26, 1, 1, n, d, "bf16", backward=True)
    mask = inputs.random_block_mask(27, nb, 0.3, True)
    mask[5, :] = 0
    mask[:, 9] = 0
    scale = api.default_scale(d)
    tm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda:0")
    tq, tk, tv, tdo = dev(q, BF), dev(k, BF), dev(v, BF), dev(do, BF)
    o, lse = api.forward_blocksparse(tq, tk, tv, tm, scale, True)
    dq, dk, dv = api.backward(tq, tk, tv, o, lse, tdo, scale, True, grad_dtype=BF, block_mask=tm)
    torch.cuda.synchronize()
    ro, rl = oracle.forward(q, k, v, scale, True, mask, inputs.MASK_BLOCK)
    rq, rk, rv = oracle.backward(q, k, v, do, scale, True, mask, inputs.MASK_BLOCK)
    errs = dict(o=max_err(host(o), ro), lse=max_err(host(lse), rl), dq=max_err(host(dq), rq),
                dk=max_err(host(dk), rk), dv=max_err(host(dv), rv))
    report(f"sparse N={n} d={d} bf16 gradients", **errs)
    assert errs["o"] <= TOL_BF16 and errs["lse"] <= TOL_LSE
    ratios = [bf16_store_ratio(host(g), r) for g, r in ((dq, rq), (dk, rk), (dv, rv))]
    report(f"sparse N={n} d={d} bf16 gradients, over the bf16-store gate", dq=ratios[0], dk=ratios[1], dv=ratios[2])
    assert max(ratios) <= 1.0, ratios


def test_autograd_wrapper_with_block_mask():
    """api.attention with a block mask: the forward and the gradients equal the explicit
    fa_fwd_ex / fa_bwd_ex calls with the mask and o_lo (bf16 gradients), and the oracle."""
    n, d = 300, 64
    nb = -(-n // 128)
    announce("autograd wrapper, block-sparse")
    q, k, v, do = inputs.random_case(28, 1, 2, n, d, "bf16", backward=True)
    mask = inputs.random_block_mask(29, nb, 0.5, True)
    tm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda:0")
    tq, tk, tv = (dev(x, BF).requires_grad_(True) for x in (q, k, v))
    out = api.attention(tq, tk, tv, None, True, tm)
    out.backward(dev(do, BF))
    o, lse, o_lo = api.forward_train(tq.detach(), tk.detach(), tv.detach(), None, True, block_mask=tm)
    eq = api.backward(tq.detach(), tk.detach(), tv.detach(), o, lse, dev(do, BF), None, True, grad_dtype=BF,
                      block_mask=tm, o_lo=o_lo)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o)
    for g, e in zip((tq.grad, tk.grad, tv.grad), eq):
        assert torch.equal(g, e)
    scale = api.default_scale(d)
    rq, rk, rv = oracle.backward(q, k, v, do, scale, True, mask, inputs.MASK_BLOCK)
    for g, r in ((tq.grad, rq), (tk.grad, rk), (tv.grad, rv)):  # bf16 gradients
        assert bf16_store_ratio(host(g), r) <= 1.0


def test_blocksparse_64k_backward_sampled():
    """The block-sparse 64K workload's backward in the launch configuration the benchmark times
    (fa_fwd_ex with o_lo, then fa_bwd_ex with the mask; fp32 gradients): dQ of 256 sampled query
    rows and dK, dV of 256 sampled keys (the boundary rows and keys included) of four heads
    against the oracle's sampled backward, which sums each key's gradient over every query
    that sees it."""
    w = inputs.WORKLOADS["blocksparse_s64k"]
    announce(w.name + " backward, sampled rows and keys of four heads")
    q, k, v, _ = inputs.make_qkv(w)
    do = inputs.draw(w.index, inputs.SLOT_DO, w.shape)
    nb = w.N // inputs.MASK_BLOCK
    mask = inputs.make_block_mask(nb, w.density, w.index, causal=w.causal)
    tq, tk, tv, tdo = dev(q, BF), dev(k, BF), dev(v, BF), dev(do, BF)
    tm = torch.from_numpy(mask).to(tq.device)
    o, lse, o_lo = api.forward_train(tq, tk, tv, w.scale, w.causal, block_mask=tm)
    ws = torch.empty(api.bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=tq.device)
    dq, dk, dv = api.backward(tq, tk, tv, o, lse, tdo, w.scale, w.causal, workspace=ws, block_mask=tm, o_lo=o_lo)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(w.N, w.sample_rows, w.index)
    keys = inputs.sample_rows(w.N, w.sample_rows, w.index, head=1)
    ri, ki = torch.from_numpy(rows).to(tq.device), torch.from_numpy(keys).to(tq.device)
    gq, gk, gv = host(dq[:, :, ri]), host(dk[:, :, ki]), host(dv[:, :, ki])
    assert np.all(np.isfinite(gq)) and np.all(np.isfinite(gk)) and np.all(np.isfinite(gv))
    errs = {}
    for b, h in ((0, 0), (0, 9), (1, 6), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.backward_rows(q[sl], k[sl], v[sl], do[sl], w.scale, w.causal, mask, inputs.MASK_BLOCK,
                                          rows=rows, keys=keys)
        errs[f"dq_{b}{h}"] = max_err(gq[sl], rq)
        errs[f"dk_{b}{h}"] = max_err(gk[sl], rk)
        errs[f"dv_{b}{h}"] = max_err(gv[sl], rv)
    report(w.name + " backward", **errs)
    assert max(errs.values()) <= TOL_BF16, errs
