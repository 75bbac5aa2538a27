"""fa_bwd_noalloc (the library's static device workspace) against fa_bwd_ex (a caller workspace).

Called through the C ABI with ctypes.  Two calls in a row on the same GPU, the second
smaller (and with grouped heads and a block mask), so the second reuses the array the
first left behind; each is compared bit for bit with fa_bwd_ex on the same inputs and
with the oracle at the bf16 tolerance.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from exact_attention_35_amd import _lib, api, inputs
from gpu_util import TOL_BF16, announce, dev, host, max_err, report

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _run_case(seed, B, H, hkv, N, d, causal, masked):
    announce(f"fa_bwd_noalloc B={B} H={H} H_kv={hkv} N={N} d={d} causal={causal} masked={masked}")
    q, k, v, do = inputs.random_case(seed, B, H, N, d, "bf16", mult=1.3, backward=True, h_kv=hkv)
    scale = api.default_scale(d)
    tq, tk, tv, tdo = dev(q, BF), dev(k, BF), dev(v, BF), dev(do, BF)
    mask_np, tm = None, None
    if masked:
        mask_np = inputs.random_block_mask(seed, -(-N // 128), 0.5, causal)
        tm = torch.from_numpy(mask_np).to(tq.device)
    o, lse, o_lo = api.forward_train(tq, tk, tv, scale, causal, block_mask=tm)
    ref = api.backward(tq, tk, tv, o, lse, tdo, scale, causal, block_mask=tm, o_lo=o_lo)
    dq, dk, dv = torch.empty_like(tq, dtype=torch.float32), torch.empty_like(tk, dtype=torch.float32), \
        torch.empty_like(tv, dtype=torch.float32)
    lib = _lib.load()
    st = lib.fa_bwd_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), None if tm is None else tm.data_ptr(),
                            o.data_ptr(), o_lo.data_ptr(), lse.data_ptr(), tdo.data_ptr(), dq.data_ptr(),
                            dk.data_ptr(), dv.data_ptr(), B, H, hkv, N, d, ctypes.c_float(scale), int(causal),
                            _lib.FA_BF16, _lib.FA_F32, torch.cuda.current_stream().cuda_stream)
    assert st == _lib.FA_OK, _lib.status_string(st)
    torch.cuda.synchronize()
    for got, want in zip((dq, dk, dv), ref):
        assert torch.equal(got, want)
    rq, rk, rv = oracle.backward(q, k, v, do, scale, causal, block_mask=mask_np)
    e = dict(dq=max_err(host(dq), rq), dk=max_err(host(dk), rk), dv=max_err(host(dv), rv))
    report(f"noalloc N={N} d={d} H_kv={hkv}", **e)
    assert max(e.values()) <= TOL_BF16, e


def test_two_calls_in_a_row_second_smaller():
    _run_case(61, 2, 4, 4, 1500, 128, True, False)
    _run_case(62, 1, 4, 2, 300, 64, False, True)


def test_through_the_binding():
    """api.backward_noalloc writes the same gradients as api.backward."""
    announce("backward_noalloc binding")
    q, k, v, do = inputs.random_case(63, 1, 2, 700, 64, "bf16", backward=True)
    tq, tk, tv, tdo = dev(q, BF), dev(k, BF), dev(v, BF), dev(do, BF)
    o, lse, o_lo = api.forward_train(tq, tk, tv, None, True)
    ref = api.backward(tq, tk, tv, o, lse, tdo, None, True, grad_dtype=BF, o_lo=o_lo)
    out = [torch.empty_like(tq) for _ in range(3)]
    api.backward_noalloc(tq, tk, tv, o, lse, tdo, *out, None, True, o_lo=o_lo)
    torch.cuda.synchronize()
    for got, want in zip(out, ref):
        assert torch.equal(got, want)
