"""The C ABI as a C program sees it: exact_attention_35_amd/fa_c_caller (built next to
libfa.so by build()) allocates its own device buffers, calls fa_fwd and fa_bwd, and
writes the results to a file, which is compared here with the fp64 oracle."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from exact_attention_35_amd import inputs
from gpu_util import TOL_BF16, TOL_LSE, announce, max_err, report

pytestmark = pytest.mark.gpu

CALLER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "exact_attention_35_amd",
                      "fa_c_caller")


def _bf16_bits(x):
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_c_program_forward_backward(tmp_path, d, causal):
    if not os.path.exists(CALLER):
        pytest.fail("fa_c_caller is not built (run build())")
    B, H, N = 2, 3, 333
    announce(f"C caller B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v, do = inputs.random_case(77 + d, B, H, N, d, "bf16", backward=True)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    np.concatenate([_bf16_bits(a).ravel() for a in (q, k, v, do)]).tofile(src)
    res = subprocess.run([CALLER, str(src), str(dst), str(B), str(H), str(N), str(d), str(int(causal))],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "d=96: -2 " in res.stdout, res.stdout  # FA_ERR_UNSUPPORTED, reported by the library
    n = B * H * N * d
    raw = dst.read_bytes()
    assert len(raw) == 2 * n + 4 * (B * H * N + 3 * n)
    o = (np.frombuffer(raw[:2 * n], dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    rest = np.frombuffer(raw[2 * n:], dtype=np.float32)
    lse, dq, dk, dv = np.split(rest, [B * H * N, B * H * N + n, B * H * N + 2 * n])
    shp = (B, H, N, d)
    scale = 1.0 / np.sqrt(d)
    ro, rl = oracle.forward(q, k, v, scale, causal)
    rdq, rdk, rdv = oracle.backward(q, k, v, do, scale, causal)
    errs = dict(o=max_err(o.reshape(shp), ro), lse=max_err(lse.reshape(shp[:3]), rl),
                dq=max_err(dq.reshape(shp), rdq), dk=max_err(dk.reshape(shp), rdk), dv=max_err(dv.reshape(shp), rdv))
    report(f"C caller d={d} causal={causal}", **errs)
    assert errs["lse"] <= TOL_LSE
    assert max(errs[k_] for k_ in ("o", "dq", "dk", "dv")) <= TOL_BF16
