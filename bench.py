#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

One step = fa_fwd_ex + fa_bwd_ex (the forward also writes the low-order part of
O, from which the recompute backward forms D) over one batch of the
long-context causal workload: B=1, H=16, N=16384, d=128, bf16, Q and K drawn as
1.7 * N(0, 1), V and dO as N(0, 1) (the Path-X length from the FlashAttention
abstract).  Inputs are resident in HBM before the timed region.

FLOPs are algorithmic: forward 4*B*H*N^2*d, halved under causal masking;
backward 2.5x the forward (five N x N x d contractions against two).
Prints one JSON line (metric, value, roofline of the dominant kernel, oracle
CPU baseline).  Run `python bench.py --help` for options.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 4096 dense bf16 flop/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2   # twice the bf16 rate (dense e4m3 MFMA)
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak, N=512-64K, d=64/128"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_s16k_d128")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the fp64 oracle")
    ap.add_argument("--no-extra", action="store_true", help="skip the per-workload kernel table")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: fwd/bwd TFLOP/s over N = 512..64K, d = 64/128, causal 0/1 "
                         "(H = 16, B = max(1, 32768 / N)), printed as one JSON line")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="print a text summary of the rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--only", choices=["step", "fwd", "bwd", "copy", "fp8"], default="step",
                    help="time only one direction (for profiling runs); 'copy' times a plain 512 MiB "
                         "device-to-device copy, the calibration kernel for the HBM byte counters; 'fp8' "
                         "times the FP8 path (quantisation of Q, K, V and the FP8 forward) and prints its table")
    return ap.parse_args()


def flops_fwd(w, density=None):
    rho = density if density is not None else (0.5 if w.causal else 1.0)
    return 4.0 * w.B * w.H * w.N * w.N * w.d * rho


def sparse_density(mask):
    import numpy as np

    nb = mask.shape[0]
    diag = int(np.trace(mask))
    off = int(mask.sum()) - diag
    return (off + 0.5 * diag) / float(nb * nb)


def to_dev(x, dtype):
    import torch

    return torch.from_numpy(x).to(dtype).to("cuda:0")


def time_launches(fn, n, warmup=2, flush=None):
    """Sorted per-launch times (ms): HIP events around each of n back-to-back calls on the
    stream (one synchronisation at the end, so the GPU never idles between them); `flush`
    is enqueued, untimed, before each call."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s, e in ev:
        if flush is not None:
            flush()
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return sorted(s.elapsed_time(e) for s, e in ev)


def gemm_reference(n=8192, reps=20):
    """bf16 GEMM n x n x n through torch (hipBLASLt): a clock-honest reference rate for the
    matrix cores under a sustained load on this machine (context for the fraction of peak)."""
    import torch

    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
    ts = time_launches(lambda: torch.matmul(a, b, out=c), reps, warmup=10)
    med = ts[len(ts) // 2]
    return {"shape": [n, n, n], "median_ms": round(med, 4), "tflops": round(2.0 * n ** 3 / med / 1e9, 1)}


def time_calls(fn, n, warmup=2):
    """Average duration (ms) of fn() measured with HIP events on torch's current stream."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    return sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / n


def kernel_table():
    """Forward/backward time and TFLOP/s of every bf16 workload (context; not the headline)."""
    import numpy as np
    import torch

    from exact_attention_35_amd import api, inputs

    rows = {}
    for name, w in inputs.WORKLOADS.items():
        if w.dtype != "bf16":
            continue
        q, k, v, _ = inputs.make_qkv(w)
        tq, tk, tv = to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16)
        del q, k, v
        entry = {"shape": list(w.shape), "causal": w.causal}
        if w.Hkv is not None:
            entry["kv_heads"] = w.kv_heads
        if w.sparse:
            nb = -(-w.N // inputs.MASK_BLOCK)
            mask = inputs.make_block_mask(nb, w.density, w.index, causal=w.causal)
            dens = sparse_density(mask)
            tm = torch.from_numpy(mask).to("cuda:0")
            ms = time_calls(lambda: api.forward_blocksparse(tq, tk, tv, tm, w.scale, w.causal), 10)
            entry.update(fwd_ms=ms, fwd_tflops=flops_fwd(w, dens) / ms / 1e9, density=dens)
            ts = time_launches(lambda: api.forward_blocksparse(tq, tk, tv, tm, w.scale, w.causal), 10)
            entry.update(fwd_median_ms=ts[len(ts) // 2], fwd_min_ms=ts[0],
                         fwd_median_frac_peak=flops_fwd(w, dens) / ts[len(ts) // 2] / 1e9 / PEAK_BF16_TFLOPS)
            # block-sparse backward on the same mask (D formed from o + o_lo, as in training)
            o, lse, o_lo = api.forward_train(tq, tk, tv, w.scale, w.causal, block_mask=tm)
            tdo = to_dev(inputs.draw(w.index, inputs.SLOT_DO, w.shape), torch.bfloat16)
            ws = torch.empty(api.bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda:0")
            bfn = lambda: api.backward(tq, tk, tv, o, lse, tdo, w.scale, w.causal, workspace=ws,  # noqa: E731
                                       block_mask=tm, o_lo=o_lo)
            bms = time_calls(bfn, 5)
            entry.update(bwd_ms=bms, bwd_tflops=2.5 * flops_fwd(w, dens) / bms / 1e9)
            bts = time_launches(bfn, 5)
            entry.update(bwd_median_ms=bts[len(bts) // 2], bwd_min_ms=bts[0],
                         bwd_median_frac_peak=2.5 * flops_fwd(w, dens) / bts[len(bts) // 2] / 1e9 / PEAK_BF16_TFLOPS)
            del o, lse, o_lo, tdo, ws
        else:
            ms = time_calls(lambda: api.forward(tq, tk, tv, w.scale, w.causal), 20)
            entry.update(fwd_ms=ms, fwd_tflops=flops_fwd(w) / ms / 1e9)
            ts = time_launches(lambda: api.forward(tq, tk, tv, w.scale, w.causal), 20)
            entry.update(fwd_median_ms=ts[len(ts) // 2], fwd_min_ms=ts[0])
            if w.N <= 1024:
                # the inputs fit in the 256 MB last-level cache: also time each launch after
                # writing a 512 MB buffer, so that they come from HBM
                junk = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
                tc = time_launches(lambda: api.forward(tq, tk, tv, w.scale, w.causal), 10,
                                   flush=lambda: junk.fill_(1))
                entry.update(fwd_cold_median_ms=tc[len(tc) // 2],
                             fwd_cold_tflops=flops_fwd(w) / tc[len(tc) // 2] / 1e9)
                del junk
                # launch-bound at this size: 10 forwards captured in one HIP graph and replayed
                o_g = torch.empty_like(tq)
                l_g = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    api.forward(tq, tk, tv, w.scale, w.causal, out=o_g, lse_out=l_g)
                torch.cuda.current_stream().wait_stream(side)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for _ in range(10):
                        api.forward(tq, tk, tv, w.scale, w.causal, out=o_g, lse_out=l_g)
                gms = time_calls(graph.replay, 10) / 10
                entry.update(fwd_graph_ms=gms, fwd_graph_tflops=flops_fwd(w) / gms / 1e9)
                del graph, o_g, l_g
            if w.backward or w.name == "long_s16k_d128" or w.Hkv is not None:
                o, lse, o_lo = api.forward_train(tq, tk, tv, w.scale, w.causal)
                tdo = to_dev(inputs.draw(w.index, inputs.SLOT_DO, w.shape), torch.bfloat16)
                ws = torch.empty(api.bwd_workspace_size(w.B, w.H, w.N, w.d, H_kv=w.kv_heads), dtype=torch.uint8,
                                 device="cuda:0")
                bfn = lambda: api.backward(tq, tk, tv, o, lse, tdo, w.scale, w.causal, workspace=ws,  # noqa: E731
                                           o_lo=o_lo)
                bms = time_calls(bfn, 10)
                entry.update(bwd_ms=bms, bwd_tflops=2.5 * flops_fwd(w) / bms / 1e9)
                bts = time_launches(bfn, 10)
                entry.update(bwd_median_ms=bts[len(bts) // 2], bwd_min_ms=bts[0])
        entry["fwd_frac_peak"] = entry["fwd_tflops"] / PEAK_BF16_TFLOPS
        rows[name] = {k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in entry.items()}
        del tq, tk, tv
        torch.cuda.empty_cache()
    return rows


def fp8_table(steps=10, warmup=2):
    """The FP8 path on long_s16k_d128: quantisation with incoherent processing (Q, K rotated, V
    not), HBM-bound, and the FP8 forward, MFMA-bound (peak: dense e4m3)."""
    import torch

    from exact_attention_35_amd import api, inputs

    w = inputs.WORKLOADS["long_s16k_d128"]
    q, k, v, _ = inputs.make_qkv(w)
    tq, tk, tv = to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16)
    del q, k, v
    signs = torch.from_numpy(inputs.random_signs(w.d, w.index)).to("cuda:0")
    q8, k8, v8 = api.quantize_fp8(tq, signs), api.quantize_fp8(tk, signs), api.quantize_fp8(tv)
    qt_ms = time_calls(lambda: api.quantize_fp8(tq, signs), steps, warmup)
    qv_ms = time_calls(lambda: api.quantize_fp8(tv), steps, warmup)
    f_ms = time_calls(lambda: api.forward_fp8(*q8, *k8, *v8, w.scale, w.causal), steps, warmup)
    n = w.B * w.H * w.N * w.d
    qbytes = n * 2 + n + w.B * w.H * (-(-w.N // 128)) * 4  # bf16 in, e4m3 codes and scales out
    ff = flops_fwd(w)
    return {"workload": w.name, "shape": list(w.shape), "causal": w.causal,
            "quantize_rotated_ms": round(qt_ms, 4), "quantize_rotated_GBs": round(qbytes / qt_ms / 1e6, 1),
            "quantize_plain_ms": round(qv_ms, 4), "quantize_plain_GBs": round(qbytes / qv_ms / 1e6, 1),
            "fwd_fp8_ms": round(f_ms, 4), "fwd_fp8_tflops": round(ff / f_ms / 1e9, 1),
            "fwd_fp8_frac_fp8_peak": round(ff / f_ms / 1e9 / PEAK_FP8_TFLOPS, 4),
            "hbm_peak_GBs": PEAK_HBM_GBS, "fp8_peak_tflops": PEAK_FP8_TFLOPS}


def sweep(compact=False):
    """TFLOP/s of the training forward (fa_fwd_ex with o_lo) and backward (fa_bwd_ex), and of
    the FP8 forward, over the metric's range of sequence lengths and head dims.

    H = 16 and B = max(1, 32768 / N) heads of iid N(0, 1) bf16 activations drawn on
    the device from a seeded generator (only timed, never checked here).  compact: fewer
    launches per point and no FP8 forward (the form printed with the headline).
    """
    import torch

    from exact_attention_35_amd import api

    rows = []
    gen = torch.Generator(device="cuda:0")
    for d in (64, 128):
        for causal in (False, True):
            for N in (512, 1024, 2048, 4096, 8192, 16384, 32768, 65536):
                B, H = max(1, 32768 // N), 16
                gen.manual_seed(35 * 1000003 + N * 7 + d + int(causal))
                shape = (B, H, N, d)
                q, k, v, do = (torch.randn(shape, generator=gen, device="cuda:0", dtype=torch.float32)
                               .to(torch.bfloat16) for _ in range(4))
                o, lse, o_lo = api.forward_train(q, k, v, None, causal)
                ws = torch.empty(api.bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda:0")
                fl = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
                n_it = max(2, min(10, int(1e12 / fl))) if compact else max(3, min(20, int(2e12 / fl)))
                f_ms = time_calls(lambda: api.forward_train(q, k, v, None, causal, out=o, lse_out=lse,
                                                            o_lo_out=o_lo), n_it)
                b_ms = time_calls(lambda: api.backward(q, k, v, o, lse, do, None, causal, workspace=ws, o_lo=o_lo),
                                  n_it)
                row = {"N": N, "d": d, "causal": causal, "B": B, "H": H,
                       "fwd_ms": round(f_ms, 4), "fwd_tflops": round(fl / f_ms / 1e9, 1),
                       "fwd_frac_peak": round(fl / f_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                       "bwd_ms": round(b_ms, 4), "bwd_tflops": round(2.5 * fl / b_ms / 1e9, 1),
                       "bwd_frac_peak": round(2.5 * fl / b_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
                if not compact:
                    # FP8 forward on the same inputs (Q, K rotated), quantisation outside the timing
                    signs = torch.where(torch.rand(d, generator=gen, device="cuda:0") < 0.5, -1, 1).to(torch.int8)
                    q8, k8, v8 = api.quantize_fp8(q, signs), api.quantize_fp8(k, signs), api.quantize_fp8(v)
                    f8_ms = time_calls(lambda: api.forward_fp8(*q8, *k8, *v8, None, causal), n_it)
                    row.update(fwd_fp8_ms=round(f8_ms, 4), fwd_fp8_tflops=round(fl / f8_ms / 1e9, 1),
                               fwd_fp8_frac_fp8_peak=round(fl / f8_ms / 1e9 / PEAK_FP8_TFLOPS, 4))
                    del q8, k8, v8
                rows.append(row)
                print(f"sweep N={N} d={d} causal={causal}: fwd {row['fwd_tflops']} TFLOP/s, "
                      f"bwd {row['bwd_tflops']} TFLOP/s"
                      + ("" if compact else f", fwd fp8 {row['fwd_fp8_tflops']} TFLOP/s"),
                      file=sys.stderr, flush=True)
                del q, k, v, do, o, lse, o_lo, ws
                torch.cuda.empty_cache()
    return rows


def host_cpu():
    """Model name, physical and logical core counts, and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        import psutil

        physical = psutil.cpu_count(logical=False)
    except Exception:  # pragma: no cover
        physical = None
    try:
        allowed = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        allowed = None
    return {"model": model, "physical_cores": physical, "logical_cpus": os.cpu_count(), "allowed_cpus": allowed}


def cpu_baseline(w, min_seconds=10.0, max_heads=4):
    """The fp64 oracle, as it stands, on the first heads of the workload (forward +
    backward of heads (0, 0), (0, 1), ... until about min_seconds of CPU work)."""
    import numpy as np

    import oracle
    from exact_attention_35_amd import inputs

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q, k, v, do = inputs.make_qkv(w)
    if do is None:
        do = inputs.draw(w.index, inputs.SLOT_DO, w.shape)
    dt, heads = 0.0, 0
    while heads < min(max_heads, w.H) and (heads == 0 or dt < min_seconds):
        sl = (slice(0, 1), slice(heads, heads + 1))
        t0 = time.perf_counter()
        oracle.forward(q[sl], k[sl], v[sl], w.scale, w.causal)
        oracle.backward(q[sl], k[sl], v[sl], do[sl], w.scale, w.causal)
        dt += time.perf_counter() - t0
        heads += 1
    one_head = flops_fwd(w) / (w.B * w.H) * 3.5
    return {"value": heads * one_head / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"forward + backward of heads (0,0)..(0,{heads - 1}) of {w.name} [N={w.N}, d={w.d}, "
                      f"causal] in fp64 NumPy, {dt:.1f} s; algorithmic flops of those heads",
            "cores_meaning": "BLAS threads the oracle ran with", "cpu": host_cpu()}


COPY_BYTES = 512 << 20

# HBM traffic per launch of fa_fwd and fa_bwd on long_s16k_d128, from separate
# rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs (KiB per dispatch, summed
# over the kernels of one call), each scaled by what the same counter reads for
# the COPY_BYTES calibration copy (FETCH_SIZE reads half of the copied bytes,
# WRITE_SIZE all of them).  A figure holds only for the sources it was taken
# on: when their hash differs the traffic is reported as null.
TRAFFIC_FETCH_SCALE = 2.0
TRAFFIC_WRITE_SCALE = 1.0
MEASURED_TRAFFIC = {
    # fwd_bf16_kernel writing o, o_lo and lse (fa_fwd_ex)
    "fwd": {"fetch_kib": 247409.1, "write_kib": 133150.1,
            "sources": ["fa_fwd.hip", "fa_device.hpp", "fa_tiles.hpp"],
            "sha256": "285cca64868389f10df88a08b658ece7a4b8c8d79deddfab7ef370505cc3f434"},
    # bwd_dq_kernel (also reading o, o_lo for D) + bwd_dkdv_kernel (fa_bwd_ex)
    "bwd": {"fetch_kib": 389220.5 + 363384.7, "write_kib": 133120.0 + 262144.0,
            "sources": ["fa_bwd.hip", "fa_device.hpp", "fa_tiles.hpp"],
            "sha256": "d26a4711fd58490c537e25e32f13b5cb77aa70b2c58ffe0d056d1939bbecb7d4"},
}


def sources_sha256(names):
    """sha256 of the sources with comments and blank lines removed (a comment edit
    does not change the kernels the figures were measured on)."""
    import hashlib
    import re

    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_attention_35_amd", "csrc", n), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [l.rstrip() for l in text.splitlines() if l.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()


def measured_traffic(which):
    """HBM bytes per launch of the forward or backward kernel, or None when stale."""
    m = MEASURED_TRAFFIC[which]
    if sources_sha256(m["sources"]) != m["sha256"]:
        return None
    return m["fetch_kib"] * 1024 * TRAFFIC_FETCH_SCALE + m["write_kib"] * 1024 * TRAFFIC_WRITE_SCALE


def profile_summary(d):
    """Text summary of a rocprofv3 output tree (CSV files, or the SQLite results database):
    kernel-trace stats and PMC counters per dispatch."""
    import csv
    import glob
    import sqlite3
    from collections import defaultdict

    lines = []
    def query(con, sql):
        try:
            return con.execute(sql).fetchall()
        except sqlite3.OperationalError:  # a results database without that view
            return []

    for f in sorted(glob.glob(os.path.join(d, "**", "*results.db"), recursive=True)):
        con = sqlite3.connect(f)
        rows = query(con, "select name, duration from kernels")
        if rows:
            per = defaultdict(list)
            for name, dur in rows:
                per[name].append(dur / 1e3)
            total = sum(sum(v) for v in per.values())
            lines.append(f"kernel-trace stats ({os.path.relpath(f, d)}):")
            lines.append(f"  {'calls':>5} {'avg us':>10} {'median us':>10} {'min us':>10} {'max us':>10} {'%':>6}  kernel")
            for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
                sv = sorted(v)
                lines.append(f"  {len(v):>5} {sum(v) / len(v):10.1f} {sv[len(sv) // 2]:10.1f} {sv[0]:10.1f} "
                             f"{sv[-1]:10.1f} {100.0 * sum(v) / total:6.2f}  {name[:90]}")
        crow = query(con, "select dispatch_id, kernel_name, counter_name, value from counters_collection")
        if crow:
            disp = defaultdict(float)
            names = {}
            for did, kname, cname, val in crow:
                disp[(did, cname)] += val
                names[did] = kname
            agg = defaultdict(list)
            for (did, cname), val in disp.items():
                agg[(cname, names[did])].append(val)
            lines.append(f"pmc ({os.path.relpath(f, d)}):")
            for (c, k), v in agg.items():
                unit = " KiB" if c in ("FETCH_SIZE", "WRITE_SIZE") else ""
                lines.append(f"  {c:>10} {len(v):3d} dispatches, mean {sum(v) / len(v):16.1f}{unit}  {k[:90]}")
        con.close()
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        lines.append(f"kernel-trace stats ({os.path.relpath(f, d)}):")
        lines.append(f"  {'calls':>5} {'avg us':>10} {'min us':>10} {'max us':>10} {'%':>6}  kernel")
        for r in csv.DictReader(open(f)):
            lines.append(f"  {r['Calls']:>5} {float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
                         f"{float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):6.2f}  {r['Name'][:90]}")
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        agg = defaultdict(list)
        for r in csv.DictReader(open(f)):
            agg[(r["Counter_Name"], r["Kernel_Name"])].append(float(r["Counter_Value"]))
        lines.append(f"pmc ({os.path.relpath(f, d)}):")
        for (c, k), v in agg.items():
            unit = " KiB" if c in ("FETCH_SIZE", "WRITE_SIZE") else ""
            lines.append(f"  {c:>10} {len(v):3d} dispatches, mean {sum(v) / len(v):16.1f}{unit}  {k[:90]}")
    return "\n".join(lines)


def copy_calibration(args):
    """A plain device copy of COPY_BYTES: its FETCH_SIZE / WRITE_SIZE counters per
    dispatch, against the known byte count, give the scale of those counters."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms = time_calls(lambda: dst.copy_(src), args.steps, args.warmup)
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "ms": round(ms, 4),
                      "GB_per_s": round(2 * COPY_BYTES / ms / 1e6, 1)}), flush=True)


def main():
    args = parse()
    if args.profile_summary:
        print(profile_summary(args.profile_summary))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from exact_attention_35_amd import api, inputs

    if args.sweep:
        print(json.dumps({"metric": METRIC, "unit": "TFLOP/s", "dtype": "bf16", "data": "synthetic",
                          "peak": PEAK_BF16_TFLOPS, "sweep": sweep()}), flush=True)
        return
    if args.only == "copy":
        copy_calibration(args)
        return
    if args.only == "fp8":
        print(json.dumps({"fp8": fp8_table(args.steps, args.warmup)}), flush=True)
        return
    w = inputs.WORKLOADS[args.workload]
    assert w.dtype == "bf16", "the step times a bf16 workload"
    q, k, v, _ = inputs.make_qkv(w)
    do = inputs.draw(w.index, inputs.SLOT_DO, w.shape)
    bf = torch.bfloat16
    tq, tk, tv, tdo = to_dev(q, bf), to_dev(k, bf), to_dev(v, bf), to_dev(do, bf)
    del q, k, v, do
    o = torch.empty_like(tq)
    o_lo = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(api.bwd_workspace_size(w.B, w.H, w.N, w.d, H_kv=w.kv_heads), dtype=torch.uint8,
                     device="cuda:0")
    density, tm = None, None
    if w.sparse:  # the block-sparse workload: its tile mask, and flops scaled by its density
        mask = inputs.make_block_mask(-(-w.N // inputs.MASK_BLOCK), w.density, w.index, causal=w.causal)
        density = sparse_density(mask)
        tm = torch.from_numpy(mask).to("cuda:0")

    do_fwd = args.only in ("step", "fwd")
    do_bwd = args.only in ("step", "bwd")
    if not do_fwd:
        api.forward_train(tq, tk, tv, w.scale, w.causal, block_mask=tm, out=o, lse_out=lse, o_lo_out=o_lo)

    def step(ev=None):
        if do_fwd:
            if ev is not None:
                ev[0].record()
            api.forward_train(tq, tk, tv, w.scale, w.causal, block_mask=tm, out=o, lse_out=lse, o_lo_out=o_lo)
            if ev is not None:
                ev[1].record()
        if do_bwd:
            if ev is not None:
                ev[2].record()
            api.backward(tq, tk, tv, o, lse, tdo, w.scale, w.causal, workspace=ws, block_mask=tm, o_lo=o_lo)
            if ev is not None:
                ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    f_fwd = flops_fwd(w, density)
    f_bwd = 2.5 * f_fwd
    f_step = (f_fwd if do_fwd else 0.0) + (f_bwd if do_bwd else 0.0)
    fwd_all = [e[0].elapsed_time(e[1]) for e in events] if do_fwd else None
    bwd_all = [e[2].elapsed_time(e[3]) for e in events] if do_bwd else None
    step_all = [e[0 if do_fwd else 2].elapsed_time(e[3 if do_bwd else 1]) for e in events]
    fwd_ms = float(np.mean(fwd_all)) if do_fwd else None
    bwd_ms = float(np.mean(bwd_all)) if do_bwd else None
    value = f_step * args.steps / elapsed / 1e12

    def spread(ts):
        return None if ts is None else {"mean": round(float(np.mean(ts)), 4), "median": round(float(np.median(ts)), 4),
                                        "min": round(float(np.min(ts)), 4), "max": round(float(np.max(ts)), 4)}

    # dominant launch by time: fa_bwd (its kernels bwd_dq and bwd_dkdv run back to
    # back on the stream and are timed together, as one launch of the backward) or
    # fa_fwd (one kernel, fwd_bf16_kernel)
    if do_bwd and (not do_fwd or bwd_ms >= fwd_ms):
        dom, dom_ms, dom_flops, which = "fa_bwd_ex (bwd_dq + bwd_dkdv)", bwd_ms, f_bwd, "bwd"
    else:
        dom, dom_ms, dom_flops, which = "fa_fwd_ex (fwd_bf16_kernel)", fwd_ms, f_fwd, "fwd"
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic = measured_traffic(which) if w.name == "long_s16k_d128" else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic), "kernel": dom,
                "launch_ms": round(dom_ms, 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "kv_heads": w.kv_heads, "block_sparse_density": density,
                   "step": {"step": "fa_fwd_ex + fa_bwd_ex (with o_lo)", "fwd": "fa_fwd_ex",
                            "bwd": "fa_bwd_ex"}[args.only],
                   "parallelism": "none (one GPU)"},
        "fwd": None if fwd_ms is None else {"ms": round(fwd_ms, 4), "tflops": round(f_fwd / fwd_ms / 1e9, 2),
                                            "frac_peak": round(f_fwd / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4)},
        "bwd": None if bwd_ms is None else {"ms": round(bwd_ms, 4), "tflops": round(f_bwd / bwd_ms / 1e9, 2),
                                            "frac_peak": round(f_bwd / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4)},
        "roofline": roofline,
        # per-step spread (HIP events around each launch); the step is forward + backward
        "ms_spread": {"step": spread(step_all), "fwd": spread(fwd_all), "bwd": spread(bwd_all),
                      "step_tflops_at_median": round(f_step / float(np.median(step_all)) / 1e9, 2)},
    }
    if not args.no_extra and args.only == "step":
        del tq, tk, tv, tdo, o, lse, o_lo, ws, tm
        torch.cuda.empty_cache()
        # the metric's range: training forward and backward over N = 512..64K, d = 64/128, causal 0/1
        out["sweep"] = sweep(compact=True)
        out["workloads"] = kernel_table()
        out["fp8"] = fp8_table()
        g = gemm_reference()
        g["fwd_frac_of_gemm"] = None if fwd_ms is None else round(f_fwd / fwd_ms / 1e9 / g["tflops"], 4)
        g["bwd_frac_of_gemm"] = None if bwd_ms is None else round(f_bwd / bwd_ms / 1e9 / g["tflops"], 4)
        out["gemm_reference"] = g
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
