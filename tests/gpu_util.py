"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""

import sys

import numpy as np
import torch

TOL_F32 = 1e-5   # max |GPU - oracle| for fp32 inputs
TOL_BF16 = 2e-2  # max |GPU - oracle| for bf16 inputs with fp32 accumulation
TOL_LSE = 1e-3   # max |GPU - oracle| of the row log-sum-exp

DEV = "cuda:0"


def dev(x, dtype):
    """float32 numpy (already bf16-representable for bf16) -> device tensor, exactly."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_store_ratio(got, ref, tol=TOL_BF16):
    """max over elements of |got - ref| / (tol (1 + 2^-8) + 2^-8 |ref|): the gate of a value
    computed to within tol in fp32 and then stored in bf16, whose rounding adds at most half
    an ulp, 2^-8 of the value (8 significant bits).  <= 1 passes; inf if the non-finite
    entries differ."""
    a = np.asarray(got, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    if a.size == 0:
        return 0.0
    fa, fb = np.isfinite(a), np.isfinite(b)
    if not np.array_equal(fa, fb) or not np.array_equal(a[~fa], b[~fb]):
        return float("inf")
    gate = tol * (1.0 + 2.0 ** -8) + 2.0 ** -8 * np.abs(b[fb])
    return float(np.max(np.abs(a[fa] - b[fb]) / gate, initial=0.0))


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    fa, fb = np.isfinite(a), np.isfinite(b)
    if not np.array_equal(fa, fb) or not np.array_equal(a[~fa], b[~fb]):
        return float("inf")
    return float(np.max(np.abs(a[fa] - b[fb]), initial=0.0))


def report(name, **errs):
    msg = " ".join(f"{k}={v:.3e}" for k, v in errs.items())
    print(f"[parity] {name}: {msg}", flush=True)
    sys.stdout.flush()


def announce(name):
    print(f"[gpu-case] {name}", flush=True)
