"""GPU forward parity: the HIP path (through the C ABI) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_35_amd import api, inputs
from gpu_util import TOL_BF16, TOL_F32, TOL_LSE, announce, dev, host, max_err, report

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def run_fwd(q, k, v, dtype, scale, causal):
    o, lse = api.forward(dev(q, dtype), dev(k, dtype), dev(v, dtype), scale, causal)
    torch.cuda.synchronize()
    return host(o), host(lse)


def test_tiny_f32_workload():
    w = inputs.WORKLOADS["tiny_f32"]
    announce(w.name)
    q, k, v, _ = inputs.make_qkv(w)
    o, lse = run_fwd(q, k, v, torch.float32, w.scale, w.causal)
    ro, rl = oracle.forward(q, k, v, w.scale, w.causal)
    eo, el = max_err(o, ro), max_err(lse, rl)
    report(w.name, o=eo, lse=el)
    assert eo <= TOL_F32 and el <= TOL_F32


def test_bert_large_workload():
    w = inputs.WORKLOADS["bert_large_s512"]
    announce(w.name)
    q, k, v, _ = inputs.make_qkv(w)
    o, lse = run_fwd(q, k, v, BF, w.scale, w.causal)
    ro, rl = oracle.forward(q, k, v, w.scale, w.causal)
    eo, el = max_err(o, ro), max_err(lse, rl)
    report(w.name, o=eo, lse=el)
    assert eo <= TOL_BF16 and el <= TOL_LSE


def test_long_16k_workload_sampled_rows():
    w = inputs.WORKLOADS["long_s16k_d128"]
    announce(w.name)
    q, k, v, _ = inputs.make_qkv(w)
    o, lse = run_fwd(q, k, v, BF, w.scale, w.causal)
    rows = inputs.sample_rows(w.N, w.sample_rows, w.index)
    ro, rl = oracle.forward_rows(q, k, v, rows, w.scale, w.causal)
    eo, el = max_err(o[:, :, rows], ro), max_err(lse[:, :, rows], rl)
    report(w.name, o=eo, lse=el, rows=float(rows.size))
    assert eo <= TOL_BF16 and el <= TOL_LSE
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_million_token_sequence_sampled_rows():
    """A long single head: N = 2^20 + 77 (a ragged tail), d = 64, causal, bf16 (8193 query
    blocks, up to 16K key tiles per workgroup, 128 MB per input): 40 sampled rows against the
    oracle, including the first, the last and the rows around the tail."""
    n, d = (1 << 20) + 77, 64
    announce(f"fwd bf16 N={n} d={d} causal")
    q, k, v, _ = inputs.random_case(29, 1, 1, n, d, "bf16")
    scale = api.default_scale(d)
    o, lse = api.forward(dev(q, BF), dev(k, BF), dev(v, BF), scale, True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([inputs.sample_rows(n, 32, 29), [n - 78, n - 77, n - 76, n - 2]]))
    idx = torch.from_numpy(rows).to(o.device)
    go, gl = host(o[:, :, idx]), host(lse[:, :, idx])
    ro, rl = oracle.forward_rows(q, k, v, rows, scale, True)
    eo, el = max_err(go, ro), max_err(gl, rl)
    report(f"N={n} d={d} causal", o=eo, lse=el, rows=float(rows.size))
    assert eo <= TOL_BF16 and el <= TOL_LSE


EDGE_N = [1, 2, 17, 64, 127, 128, 129, 300, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths_bf16(d, causal):
    for n in EDGE_N:
        announce(f"fwd bf16 N={n} d={d} causal={causal}")
        q, k, v, _ = inputs.random_case(1, 2, 3, n, d, "bf16", mult=1.5)
        scale = api.default_scale(d)
        o, lse = run_fwd(q, k, v, BF, scale, causal)
        ro, rl = oracle.forward(q, k, v, scale, causal)
        eo, el = max_err(o, ro), max_err(lse, rl)
        report(f"N={n} d={d} causal={causal}", o=eo, lse=el)
        assert eo <= TOL_BF16 and el <= TOL_LSE, (n, d, causal)


@pytest.mark.parametrize("d", [64, 128])
def test_causal_around_short_sequence_limit(d):
    """Causal sequences of up to 2048 keys run on the 128-query, 4-wave forward kernel and, on
    this small grid, longer ones on the 256-query, 8-wave kernel: both sides of that limit,
    with ragged tails.
    The train-mode forward (with the low-order part of O) must give the same o and lse bit for
    bit, and o + o_lo must stay within half the bf16 tolerance of the oracle."""
    scale = api.default_scale(d)
    for n in (2047, 2048, 2049, 2177):
        announce(f"fwd bf16 causal N={n} d={d}")
        q, k, v, _ = inputs.random_case(37, 1, 2, n, d, "bf16", mult=1.5)
        tq, tk, tv = dev(q, BF), dev(k, BF), dev(v, BF)
        o, lse = api.forward(tq, tk, tv, scale, True)
        o2, lse2, o_lo = api.forward_train(tq, tk, tv, scale, True)
        torch.cuda.synchronize()
        ro, rl = oracle.forward(q, k, v, scale, True)
        eo, el = max_err(host(o), ro), max_err(host(lse), rl)
        e_full = max_err(host(o2) + host(o_lo), ro)
        report(f"causal N={n} d={d}", o=eo, lse=el, o_plus_lo=e_full)
        assert torch.equal(o, o2) and torch.equal(lse, lse2), n
        assert eo <= TOL_BF16 and el <= TOL_LSE and e_full <= TOL_BF16 / 2, n


@pytest.mark.parametrize("b, h, n, causal", [(2, 16, 2047, True), (4, 32, 1000, True), (1, 16, 4100, True),
                                              (2, 8, 3000, False)])
def test_short_kernel_d64_64key_tiles(b, h, n, causal):
    """d = 64 forwards that take the 128-query kernel with 64-key tiles at four workgroups per
    CU: causal with N <= 8192 on grids of at least 512 blocks of 128 queries, and without
    causal masking N <= 4096 on any grid.  Ragged shapes on that path, every element against
    the oracle."""
    if causal:
        assert -(-n // 128) * b * h >= 512 and n <= 8192
    announce(f"fwd bf16 B={b} H={h} N={n} d=64 causal={causal}")
    q, k, v, _ = inputs.random_case(43, b, h, n, 64, "bf16", mult=1.5)
    scale = api.default_scale(64)
    o, lse = run_fwd(q, k, v, BF, scale, causal)
    ro, rl = oracle.forward(q, k, v, scale, causal)
    eo, el = max_err(o, ro), max_err(lse, rl)
    report(f"B={b} H={h} N={n} d=64 causal={causal}", o=eo, lse=el)
    assert eo <= TOL_BF16 and el <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths_f32(d, causal):
    for n in (1, 5, 64, 65, 200):
        announce(f"fwd f32 N={n} d={d} causal={causal}")
        q, k, v, _ = inputs.random_case(2, 1, 2, n, d, "f32")
        scale = api.default_scale(d)
        o, lse = run_fwd(q, k, v, torch.float32, scale, causal)
        ro, rl = oracle.forward(q, k, v, scale, causal)
        eo, el = max_err(o, ro), max_err(lse, rl)
        assert eo <= TOL_F32 and el <= TOL_F32, (n, d, causal, eo, el)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_scale_values(scale):
    announce(f"fwd scale={scale}")
    q, k, v, _ = inputs.random_case(3, 1, 2, 200, 64, "bf16")
    for causal in (False, True):
        o, lse = run_fwd(q, k, v, BF, scale, causal)
        ro, rl = oracle.forward(q, k, v, scale, causal)
        eo, el = max_err(o, ro), max_err(lse, rl)
        report(f"scale={scale} causal={causal}", o=eo, lse=el)
        assert eo <= TOL_BF16 and el <= TOL_LSE


def test_large_logits_rescale():
    """Q, K scaled up so that the running maximum moves many times (stresses the online rescale)."""
    announce("fwd large logits")
    q, k, v, _ = inputs.random_case(4, 1, 2, 777, 128, "bf16", mult=4.0)
    scale = api.default_scale(128)
    for causal in (False, True):
        o, lse = run_fwd(q, k, v, BF, scale, causal)
        ro, rl = oracle.forward(q, k, v, scale, causal)
        eo, el = max_err(o, ro), max_err(lse, rl)
        report(f"large logits causal={causal}", o=eo, lse=el)
        assert eo <= TOL_BF16 and el <= TOL_LSE


def test_constant_v_and_ones_column():
    announce("fwd constant V")
    q, k, _, _ = inputs.random_case(5, 1, 2, 333, 64, "bf16", mult=2.0)
    c = inputs.bf16_round(np.linspace(-3, 3, 64).astype(np.float32))
    v = np.broadcast_to(c, q.shape).copy()
    for causal in (False, True):
        o, _ = run_fwd(q, k, v, BF, 0.125, causal)
        assert max_err(o, np.broadcast_to(c, o.shape)) <= TOL_BF16
    v2 = inputs.random_case(6, 1, 2, 333, 64, "bf16")[2]
    v2[..., 7] = 1.0
    o2, _ = run_fwd(q, k, v2, BF, 0.125, True)
    assert np.max(np.abs(o2[..., 7] - 1.0)) <= 1e-2


def test_deterministic_and_permutation_invariant():
    announce("fwd determinism")
    q, k, v, _ = inputs.random_case(7, 2, 2, 520, 128, "bf16")
    tq, tk, tv = dev(q, BF), dev(k, BF), dev(v, BF)
    o1, l1 = api.forward(tq, tk, tv, 0.1, True)
    o2, l2 = api.forward(tq, tk, tv, 0.1, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    perm = np.random.default_rng(0).permutation(520)
    o3, l3 = run_fwd(q, k[:, :, perm], v[:, :, perm], BF, 0.1, False)
    o4, l4 = run_fwd(q, k, v, BF, 0.1, False)
    assert max_err(o3, o4) <= TOL_BF16 and max_err(l3, l4) <= TOL_LSE


def test_no_lse_and_guard_band():
    """lse may be NULL; outputs are written exactly within their extent."""
    announce("fwd guard band")
    B, H, N, d = 1, 2, 130, 64
    q, k, v, _ = inputs.random_case(8, B, H, N, d, "bf16")
    n_el = B * H * N * d
    buf = torch.full((n_el + 2048,), 7.0, dtype=BF, device="cuda:0")
    out = buf[1024:1024 + n_el].view(B, H, N, d)
    o, lse = api.forward(dev(q, BF), dev(k, BF), dev(v, BF), 0.125, False, with_lse=False, out=out)
    torch.cuda.synchronize()
    assert lse is None
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n_el:] == 7.0)
    ro, _ = oracle.forward(q, k, v, 0.125, False)
    assert max_err(host(out), ro) <= TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_forward_train_low_order_part(d, causal, masked):
    """fa_fwd_ex with o_lo: o is bitwise the plain forward's, |o_lo| is at most half an ulp of
    o (o is O rounded to nearest), and o + o_lo is closer to the oracle than o alone.  What
    remains in o + o_lo is the rounding of P to bf16 for the P.V product (about 5e-3 at this
    logit spread), so the gate is half the bf16 tolerance."""
    n = 1030
    announce(f"fwd_ex o_lo N={n} d={d} causal={causal} masked={masked}")
    q, k, v, _ = inputs.random_case(31, 1, 3, n, d, "bf16", mult=1.5)
    scale = api.default_scale(d)
    tq, tk, tv = dev(q, BF), dev(k, BF), dev(v, BF)
    mask = None
    if masked:
        mask_np = inputs.random_block_mask(31, -(-n // 128), 0.4, causal)
        mask = torch.from_numpy(mask_np).to(tq.device)
        o_ref, lse_ref = api.forward_blocksparse(tq, tk, tv, mask, scale, causal)
        ro, rl = oracle.forward(q, k, v, scale, causal, block_mask=mask_np)
    else:
        o_ref, lse_ref = api.forward(tq, tk, tv, scale, causal)
        ro, rl = oracle.forward(q, k, v, scale, causal)
    o, lse, o_lo = api.forward_train(tq, tk, tv, scale, causal, block_mask=mask)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    ho, hl = host(o), host(o_lo)
    ulp = np.spacing(np.abs(ho).astype(np.float32)).astype(np.float64) * 2.0 ** 16  # bf16 ulp of o
    assert np.all(np.abs(hl) <= 0.5 * ulp + 1e-30)
    e_hi, e_full = max_err(ho, ro), max_err(ho + hl, ro)
    report(f"o_lo d={d} causal={causal} masked={masked}", o=e_hi, o_plus_lo=e_full)
    assert e_full <= e_hi and e_full <= TOL_BF16 / 2
