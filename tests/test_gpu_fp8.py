"""GPU parity of the FP8 path (fa_quantize_fp8, fa_fwd_fp8) against the fp64 oracle.

Quantisation decides integer codes, so it is compared bit for bit (both sides
decide in fp32, in the same transform order).  The forward is compared with exact
attention of the dequantised inputs, element by element, within a bound built from
the kernel's arithmetic:
  * P rounded to e4m3 for P.V: the oracle's `pv_rounding_bound`;
  * the scores: one v_mfma_f32_32x32x64_f8f6f4 sums its 64 products with an error
    of at most 2^-11.2 of its largest product (measured on gfx950 with random e4m3
    operands whose magnitudes spread over e^0 .. e^8; the accumulation onto C adds
    none; AMD's documents do not state it, so test_fp8_score_accumulation_property
    checks it through the library on every run), so with d/64 chained MFMAs a score
    is off by at most
    delta_i = 2^-10 (d/64) |scale| max|q_i| max|k| (a margin of about 2 over the
    measurement); that moves lse by at most delta_i and every P by a factor within
    e^(+-delta_i), hence O by at most 2 (e^delta_i - 1) sum_j P_ij |v_j| / l_i;
  * the bf16 rounding of O and the fp32 row sums: 2^-7 |O| + 1e-4.
    |O_gpu - O| <= 1.02 (pv bound + score term) + 2^-7 |O| + 1e-4,
    |lse_gpu - lse| <= delta_i + 1e-3.
The forward tests feed both sides the oracle's own codes, so they do not depend
on the quantisation kernel.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as of8
from exact_attention_35_amd import api, inputs
from gpu_util import TOL_LSE, announce, dev, host, max_err, report

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def _case_x(seed, shape, dtype):
    rng = np.random.default_rng(np.random.SeedSequence([35, 910, seed] + list(shape)))
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-2, 2, shape[:-1] + (1,)))).astype(np.float32)
    if shape[2] > 130:
        x[0, 0, 128:256] = 0.0           # an all-zero block
    x[0, -1, 0, 3] = 2000.0              # an outlier
    return inputs.bf16_round(x) if dtype == "bf16" else x


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_bit_exact(d, dtype):
    for n in (1, 100, 300):
        for rotate in (False, True):
            name = f"fp8 quantize {dtype} N={n} d={d} rotate={rotate}"
            announce(name)
            x = _case_x(n + d, (2, 3, n, d), dtype)
            signs = inputs.random_signs(d, 7) if rotate else None
            tx = dev(x, torch.bfloat16 if dtype == "bf16" else torch.float32)
            codes, scales = api.quantize_fp8(tx, None if signs is None else _u8(signs).view(torch.int8))
            torch.cuda.synchronize()
            rc, rs = of8.quantize(x, None if signs is None else signs.astype(np.float64))
            got_c = codes.cpu().numpy()
            mism = int(np.count_nonzero(got_c != rc))
            report(name, code_mismatches=float(mism), scale_err=float(np.max(np.abs(scales.cpu().numpy() - rs))))
            assert mism == 0
            assert np.array_equal(scales.cpu().numpy(), rs)


def _fwd_case(seed, B, H, hkv, n, d, mult=1.0, rotate=False):
    rng = np.random.default_rng(np.random.SeedSequence([35, 920, seed, B, H, hkv, n, d]))
    q = inputs.bf16_round((rng.standard_normal((B, H, n, d)) * mult).astype(np.float32))
    k = inputs.bf16_round((rng.standard_normal((B, hkv, n, d)) * mult).astype(np.float32))
    v = inputs.bf16_round(rng.standard_normal((B, hkv, n, d)).astype(np.float32))
    s = inputs.random_signs(d, seed).astype(np.float64) if rotate else None
    return of8.quantize(q, s), of8.quantize(k, s), of8.quantize(v), (q, k, v)


def _gates(dq, dk, dv, ro, scale, causal, rows):
    """(O gate [B, H, R, d], lse gate [B, H, R]) of the bound in the module docstring."""
    B, H, N, d = dq.shape
    kmax = np.abs(dk).max(axis=(2, 3))                                     # [B, H_kv]
    g = H // dk.shape[1]
    qmax = np.abs(dq[:, :, rows]).max(axis=-1)                             # [B, H, R]
    delta = 2.0 ** -10 * (d / 64) * abs(scale) * qmax * np.repeat(kmax, g, axis=1)[..., None]
    # sum_j P_ij |v_j| / l_i = (exact attention of |V|), the weights of the score term
    wv, _ = oracle.forward_rows(dq, dk, np.abs(dv), rows, scale, causal)
    bound = of8.pv_rounding_bound(dq, dk, dv, scale, causal, rows) + 2.0 * np.expm1(delta)[..., None] * wv
    return 1.02 * bound + 2.0 ** -7 * np.abs(ro) + 1e-4, delta + TOL_LSE


def _check_fwd(name, q8, k8, v8, scale, causal, rows=None):
    (qc, qs), (kc, ks), (vc, vs) = q8, k8, v8
    o, lse = api.forward_fp8(_u8(qc), _f32(qs), _u8(kc), _f32(ks), _u8(vc), _f32(vs), scale, causal)
    torch.cuda.synchronize()
    dq, dk, dv = of8.dequantize(qc, qs), of8.dequantize(kc, ks), of8.dequantize(vc, vs)
    N = qc.shape[2]
    rows = np.arange(N) if rows is None else rows
    ro, rl = oracle.forward_rows(dq, dk, dv, rows, scale, causal)
    gate, lgate = _gates(dq, dk, dv, ro, scale, causal, rows)
    go = host(o)[:, :, rows]
    gl = host(lse)[:, :, rows]
    err = np.abs(go - ro)
    lerr = np.abs(gl - rl)
    report(name, o=float(err.max()), o_over_gate=float((err / gate).max()), lse=float(lerr.max()),
           lse_over_gate=float((lerr / lgate).max()))
    assert np.all(err <= gate), (name, float((err / gate).max()))
    assert np.all(lerr <= lgate), (name, float((lerr / lgate).max()))
    return go, ro


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_fp8(d, causal):
    # at d = 64, N <= 2048 runs 128-key tiles and longer sequences 256-key tiles (two K/V
    # scale blocks per tile): 2600 covers the latter with a ragged last tile
    for n in (1, 77, 300, 1000) + ((2600,) if d == 64 else ()):
        for rotate in (False, True):
            name = f"fp8 fwd N={n} d={d} causal={causal} rotate={rotate}"
            announce(name)
            q8, k8, v8, _ = _fwd_case(n, 2, 2, 2, n, d, mult=1.5, rotate=rotate)
            _check_fwd(name, q8, k8, v8, api.default_scale(d), causal)


def test_forward_fp8_gqa_and_scales():
    """Grouped-query heads, a negative scale, scale 0, and large logits (many running-max rescales)."""
    for hkv, scale, mult in ((2, None, 1.0), (1, -0.1, 1.0), (4, 0.0, 1.0), (2, None, 4.0)):
        d = 128
        sc = api.default_scale(d) if scale is None else scale
        name = f"fp8 fwd H=4 H_kv={hkv} scale={sc:.4f} mult={mult}"
        announce(name)
        q8, k8, v8, _ = _fwd_case(hkv * 10 + int(mult), 1, 4, hkv, 700, d, mult=mult, rotate=True)
        for causal in (False, True):
            _check_fwd(name + f" causal={causal}", q8, k8, v8, sc, causal)


def test_fp8_long_workload_sampled_rows():
    """The 16K, d = 128 workload quantised on the GPU with incoherent processing: every code and
    scale of Q, K and V bit-exact against the oracle, and the forward on 256 sampled rows of
    heads 0 and 15 within the bound; the error against bf16 exact attention is reported."""
    w = inputs.WORKLOADS["long_s16k_d128"]
    announce("fp8 " + w.name)
    q, k, v, _ = inputs.make_qkv(w)
    signs = inputs.random_signs(w.d, w.index)
    tsg = _u8(signs).view(torch.int8)
    tq, tk, tv = dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16)
    q8 = api.quantize_fp8(tq, tsg)
    k8 = api.quantize_fp8(tk, tsg)
    v8 = api.quantize_fp8(tv)
    torch.cuda.synchronize()
    for name, (c, s), x, sg in (("q", q8, q, signs), ("k", k8, k, signs), ("v", v8, v, None)):
        rc, rs = of8.quantize(x, None if sg is None else sg.astype(np.float64))
        mism = int(np.count_nonzero(c.cpu().numpy() != rc))
        report(f"fp8 {w.name} quantize {name}", code_mismatches=float(mism))
        assert mism == 0 and np.array_equal(s.cpu().numpy(), rs)
    rows = inputs.sample_rows(w.N, w.sample_rows // 2, w.index)
    o, lse = api.forward_fp8(*q8, *k8, *v8, w.scale, w.causal)
    torch.cuda.synchronize()
    qc, qs = (t.cpu().numpy() for t in q8)
    kc, ks = (t.cpu().numpy() for t in k8)
    vc, vs = (t.cpu().numpy() for t in v8)
    for h in (0, 15):
        sl = slice(h, h + 1)
        dq = of8.dequantize(qc[:, sl], qs[:, sl])
        dk = of8.dequantize(kc[:, sl], ks[:, sl])
        dv = of8.dequantize(vc[:, sl], vs[:, sl])
        ro, rl = oracle.forward_rows(dq, dk, dv, rows, w.scale, w.causal)
        gate, lgate = _gates(dq, dk, dv, ro, w.scale, w.causal, rows)
        go = host(o)[:, sl][:, :, rows]
        err = np.abs(go - ro)
        lerr = np.abs(host(lse)[:, sl][:, :, rows] - rl)
        exact, _ = oracle.forward_rows(q[:, sl], k[:, sl], v[:, sl], rows, w.scale, w.causal)
        rmse = float(np.sqrt(np.mean((go - exact) ** 2)))
        report(f"fp8 {w.name} head {h}", o=float(err.max()), o_over_gate=float((err / gate).max()),
               lse=float(lerr.max()), lse_over_gate=float((lerr / lgate).max()), rmse_vs_bf16_exact=rmse)
        assert np.all(err <= gate)
        assert np.all(lerr <= lgate)
        assert rmse <= 0.05


def test_incoherent_processing_on_gpu():
    """With outlier coordinates in Q and K, the GPU path with the rotation is closer to exact
    attention of the original inputs than without it."""
    announce("fp8 incoherent processing")
    rng = np.random.default_rng(np.random.SeedSequence([35, 930]))
    d, N = 128, 512
    q = rng.standard_normal((1, 2, N, d))
    k = rng.standard_normal((1, 2, N, d))
    v = rng.standard_normal((1, 2, N, d))
    q[..., :3] *= 40.0
    k[..., :3] *= 40.0
    q, k, v = (inputs.bf16_round(a.astype(np.float32)) for a in (q, k, v))
    scale = api.default_scale(d) / 4.0
    exact, _ = oracle.forward(q, k, v, scale, True)
    tq, tk, tv = (dev(a, torch.bfloat16) for a in (q, k, v))
    tsg = _u8(inputs.random_signs(d, 3)).view(torch.int8)
    v8 = api.quantize_fp8(tv)
    o_plain, _ = api.forward_fp8(*api.quantize_fp8(tq), *api.quantize_fp8(tk), *v8, scale, True)
    o_rot, _ = api.forward_fp8(*api.quantize_fp8(tq, tsg), *api.quantize_fp8(tk, tsg), *v8, scale, True)
    torch.cuda.synchronize()
    e_plain = float(np.sqrt(np.mean((host(o_plain) - exact) ** 2)))
    e_rot = float(np.sqrt(np.mean((host(o_rot) - exact) ** 2)))
    report("fp8 incoherent processing", rmse_plain=e_plain, rmse_rotated=e_rot)
    assert e_rot < 0.8 * e_plain


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_score_accumulation_property(d):
    """The score term of the forward gate rests on how v_mfma_f32_32x32x64_f8f6f4 sums its
    64 products, which AMD's documents do not state.  This checks that property through the
    library itself: a row with a single key has P = 1 and l = 1, so its lse is exactly
    |scale| times the kernel's own fp32 score (the quantisation scales are powers of two).
    With codes whose magnitudes spread over e^0 .. e^8 inside a row, the score error of
    every row must stay within 2^-10 (d/64) max|q| max|k|, the bound the gate assumes; the
    report gives the error in units of the summed largest product of each 64-product MFMA
    (2^-11.4 at d = 64 and 2^-12.1 at d = 128 on these inputs).
    """
    B, H = 16, 32
    rng = np.random.default_rng(np.random.SeedSequence([35, 930, d]))

    def spread(shape):
        return (rng.choice([-1.0, 1.0], size=shape) * np.exp(rng.uniform(0.0, 8.0, size=shape))).astype(np.float32)

    q8 = of8.quantize(spread((B, H, 1, d)))
    k8 = of8.quantize(spread((B, H, 1, d)))
    v8 = of8.quantize(spread((B, H, 1, d)))
    (qc, qs), (kc, ks), (vc, vs) = q8, k8, v8
    _, lse = api.forward_fp8(_u8(qc), _f32(qs), _u8(kc), _f32(ks), _u8(vc), _f32(vs), 1.0, False)
    torch.cuda.synchronize()
    dq = of8.dequantize(qc, qs)[:, :, 0]  # [B, H, d], exact in fp64
    dk = of8.dequantize(kc, ks)[:, :, 0]
    prod = dq * dk
    exact = prod.sum(axis=-1)
    err = np.abs(host(lse)[:, :, 0].astype(np.float64) - exact)
    chunks = prod.reshape(B, H, d // 64, 64)
    maxprod = np.abs(chunks).max(axis=-1).sum(axis=-1)              # sum over the chained MFMAs
    gate_term = 2.0 ** -10 * (d / 64) * np.abs(dq).max(-1) * np.abs(dk).max(-1)
    fp32_slack = 2.0 ** -21 * np.abs(prod).sum(axis=-1)             # the scaling multiplies after the MFMA
    ratio = float((err / maxprod).max())
    report(f"fp8 score accumulation d={d}", err_over_maxprod_log2=float(np.log2(max(ratio, 2.0 ** -40))),
           err_over_gate=float((err / (gate_term + fp32_slack)).max()))
    assert np.all(err <= gate_term + fp32_slack), float((err / (gate_term + fp32_slack)).max())


def test_forward_fp8_head_runs():
    """Without causal masking the FP8 forward's grid runs head by head on each XCD once B*H is
    a multiple of 8 and the grid has more than 1024 workgroups: B=8, H=8, N=4500, d=128 (1152
    workgroups of 256 queries).  Outputs start as NaN, so every (block, head) pair must be
    written; heads at the start, middle and end of the grid, on 128 sampled rows each, within
    the bound."""
    from exact_attention_35_amd import _lib

    B, H, N, d = 8, 8, 4500, 128
    name = f"fp8 fwd head runs B={B} H={H} N={N} d={d}"
    announce(name)
    q8, k8, v8, _ = _fwd_case(77, B, H, H, N, d)
    (qc, qs), (kc, ks), (vc, vs) = q8, k8, v8
    scale = api.default_scale(d)
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    tq, tqs, tk, tks, tv, tvs = _u8(qc), _f32(qs), _u8(kc), _f32(ks), _u8(vc), _f32(vs)
    st = _lib.load().fa_fwd_fp8(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), tqs.data_ptr(), tks.data_ptr(),
                                tvs.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H, N, d, scale, 0,
                                torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "fa_fwd_fp8")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "entries no workgroup wrote"
    rows = inputs.sample_rows(N, 128, 77)
    go_all, gl_all = host(o), host(lse)
    for b, h in ((0, 0), (3, 6), (7, 7)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        dq, dk, dv = of8.dequantize(qc[sl], qs[sl]), of8.dequantize(kc[sl], ks[sl]), of8.dequantize(vc[sl], vs[sl])
        ro, rl = oracle.forward_rows(dq, dk, dv, rows, scale, False)
        gate, lgate = _gates(dq, dk, dv, ro, scale, False, rows)
        err = np.abs(go_all[sl][:, :, rows] - ro)
        lerr = np.abs(gl_all[sl][:, :, rows] - rl)
        report(f"{name} head ({b}, {h})", o=float(err.max()), o_over_gate=float((err / gate).max()),
               lse=float(lerr.max()), lse_over_gate=float((lerr / lgate).max()))
        assert np.all(err <= gate), (b, h, float((err / gate).max()))
        assert np.all(lerr <= lgate), (b, h, float((lerr / lgate).max()))
