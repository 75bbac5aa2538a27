"""Grids whose launch order is renumbered per XCD.

Launches without causal masking (and block-sparse ones) renumber their workgroups so
that each XCD works through its heads one after the other, when B*H is a multiple of 8
and the grid has more than 1024 workgroups; causal launches up to N = 4096 with B*H a
multiple of 8 let each XCD take its heads a few at a time (longest rows first within a
group).  Shapes the other dense tests do not reach, forward (fa_fwd_ex) and backward
(fa_bwd_ex) through the C ABI, every kernel of both on a renumbered grid:

  no causal masking:
  B=16, H=16, N=1000, d=64:  forward 128-query kernel (2048 workgroups), dQ 128-query
                             kernel (2048), dK/dV on 64-key workgroups (4096);
  B=8,  H=8,  N=4500, d=128: forward 256-query kernel (1152), dQ 256-query kernel (1152),
                             dK/dV on 128-key workgroups (2304);
  causal, heads taken a few at a time:
  B=16, H=16, N=2000, d=64:  forward 128-query kernel (16 heads per group), dQ 128-query
                             kernel (16), dK/dV on 64-key workgroups (4);
  B=8,  H=8,  N=4000, d=128: forward 256-query kernel (4), dQ 256-query kernel (4),
                             dK/dV on 128-key workgroups (2).

Every output buffer starts as NaN, so a (block, head) pair that no workgroup covers
would be left NaN: all outputs must be finite.  Whole heads at the start, middle and
end of the grid are compared element by element with the fp64 oracle (bf16 tolerances,
fp32 gradients).
"""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_35_amd import _lib, api, inputs
from gpu_util import TOL_BF16, TOL_LSE, announce, dev, host, max_err, report

pytestmark = pytest.mark.gpu

BF = torch.bfloat16

CASES = [
    (16, 16, 1000, 64, False, [(0, 0), (7, 5), (15, 15)]),
    (8, 8, 4500, 128, False, [(0, 0), (3, 6), (7, 7)]),
    (16, 16, 2000, 64, True, [(0, 0), (9, 3), (15, 15)]),
    (8, 8, 4000, 128, True, [(0, 1), (4, 2), (7, 7)]),
]


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda:0")


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_H{c[1]}_N{c[2]}_d{c[3]}_causal{int(c[4])}" for c in CASES])
def test_head_runs_forward_backward(case):
    B, H, N, d, causal, heads = case
    announce(f"launch order per XCD: B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v, do = inputs.random_case(71, B, H, N, d, "bf16", backward=True)
    tq, tk, tv, tdo = dev(q, BF), dev(k, BF), dev(v, BF), dev(do, BF)
    scale = api.default_scale(d)
    o, lse, o_lo = _nan(tq.shape, BF), _nan((B, H, N), torch.float32), _nan(tq.shape, BF)
    api.forward_train(tq, tk, tv, scale, causal, out=o, lse_out=lse, o_lo_out=o_lo)
    dq, dk, dv = (_nan(tq.shape, torch.float32) for _ in range(3))
    ws = torch.empty(max(api.bwd_workspace_size(B, H, N, d), 16), dtype=torch.uint8, device="cuda:0")
    st = _lib.load().fa_bwd_ex(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), None, o.data_ptr(), o_lo.data_ptr(),
                               lse.data_ptr(), tdo.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H,
                               N, d, scale, int(causal), _lib.FA_BF16, _lib.FA_F32, ws.data_ptr(), ws.numel(),
                               torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "fa_bwd_ex")
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("o_lo", o_lo), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"{name}: entries no workgroup wrote"
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rl = oracle.forward(q[sl], k[sl], v[sl], scale, causal)
        rq, rk, rv = oracle.backward(q[sl], k[sl], v[sl], do[sl], scale, causal)
        e = dict(o=max_err(host(o[sl]), ro), lse=max_err(host(lse[sl]), rl), dq=max_err(host(dq[sl]), rq),
                 dk=max_err(host(dk[sl]), rk), dv=max_err(host(dv[sl]), rv))
        report(f"launch order B={B} H={H} N={N} d={d} causal={causal} head ({b}, {h})", **e)
        assert e["lse"] <= TOL_LSE, (b, h, e)
        assert max(e["o"], e["dq"], e["dk"], e["dv"]) <= TOL_BF16, (b, h, e)
