"""The Python binding rejects malformed caller buffers before any library call (no GPU).

The library itself is replaced by a stand-in whose compute entry points raise
`LibCalled`, and the binding's "is this tensor on a GPU" test is made to accept
CPU tensors: a well-formed call then reaches the library (LibCalled), and a
malformed one must raise ValueError first, so no kernel could ever be launched
on a wrong-sized, wrong-typed or non-contiguous buffer.
"""

import pytest
import torch

from exact_attention_35_amd import _lib, api


class LibCalled(Exception):
    pass


class FakeLib:
    """Sizes answer like the real library; any compute entry point raises LibCalled."""

    def fa_bwd_workspace_size(self, B, H, N, d, grad_dtype):
        return 8 * B * H * N

    def fa_bwd_gqa_workspace_size(self, B, H, H_kv, N, d, grad_dtype):
        return 8 * B * H * N + (0 if H_kv == H else 8 * B * H * N * d + 256)

    def __getattr__(self, name):
        def call(*args):
            raise LibCalled(name)
        return call


@pytest.fixture(autouse=True)
def fake_lib(monkeypatch):
    monkeypatch.setattr(_lib, "load", lambda: FakeLib())
    monkeypatch.setattr(api, "_on_gpu", lambda t: True)
    monkeypatch.setattr(api, "_stream_ptr", lambda device: 0)
    monkeypatch.setattr(api, "_on_device", lambda device: _NullContext())


class _NullContext:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


B, H, N, D = 1, 2, 40, 64
BF = torch.bfloat16


def qkv(dtype=BF, heads_kv=H):
    q = torch.zeros(B, H, N, D, dtype=dtype)
    k = torch.zeros(B, heads_kv, N, D, dtype=dtype)
    v = torch.zeros(B, heads_kv, N, D, dtype=dtype)
    return q, k, v


def bad_outputs(dtype=BF):
    """(name, tensor) pairs of malformed o / lse buffers."""
    return [
        ("o short", torch.zeros(B, H, N - 1, D, dtype=dtype)),
        ("o dtype", torch.zeros(B, H, N, D, dtype=torch.float16)),
        ("o strided", torch.zeros(B, H, D, N, dtype=dtype).transpose(2, 3)),
        ("o numpy", torch.zeros(B, H, N, D, dtype=dtype).numpy() if dtype != BF else [0]),
    ]


def test_well_formed_calls_reach_the_library():
    q, k, v = qkv()
    with pytest.raises(LibCalled):
        api.forward(q, k, v, out=torch.empty_like(q), lse_out=torch.empty(B, H, N))
    with pytest.raises(LibCalled):
        api.forward_train(q, k, v, out=torch.empty_like(q), lse_out=torch.empty(B, H, N),
                          o_lo_out=torch.empty_like(q))
    mask = torch.ones(1, 1, dtype=torch.uint8)
    with pytest.raises(LibCalled):
        api.forward_blocksparse(q, k, v, mask, out=torch.empty_like(q), lse_out=torch.empty(B, H, N))
    o, lse, do = torch.zeros_like(q), torch.zeros(B, H, N), torch.zeros_like(q)
    ws = torch.empty(8 * B * H * N, dtype=torch.uint8)
    with pytest.raises(LibCalled):
        api.backward(q, k, v, o, lse, do, workspace=ws)
    with pytest.raises(LibCalled):
        api.backward(q, k, v, o, lse, do, workspace=ws, o_lo=torch.zeros_like(q))


@pytest.mark.parametrize("which", ["forward", "forward_train", "forward_blocksparse"])
def test_forward_rejects_malformed_outputs(which):
    q, k, v = qkv()
    mask = torch.ones(1, 1, dtype=torch.uint8)

    def call(**kw):
        if which == "forward":
            return api.forward(q, k, v, **kw)
        if which == "forward_train":
            return api.forward_train(q, k, v, **kw)
        return api.forward_blocksparse(q, k, v, mask, **kw)

    for name, bad in bad_outputs():
        with pytest.raises(ValueError):
            call(out=bad)
    for bad in (torch.zeros(B, H, N + 1), torch.zeros(B, H, N, dtype=torch.float64),
                torch.zeros(B, H * N)[:, :].reshape(B, H, N).transpose(1, 2).contiguous().transpose(1, 2),
                torch.zeros(B, N, H).transpose(1, 2)):
        with pytest.raises(ValueError):
            call(lse_out=bad)
    if which == "forward_train":
        for name, bad in bad_outputs():
            with pytest.raises(ValueError):
                call(o_lo_out=bad)


def test_forward_lse_out_without_lse_is_rejected():
    q, k, v = qkv()
    with pytest.raises(ValueError):
        api.forward(q, k, v, with_lse=False, lse_out=torch.empty(B, H, N))


def test_forward_train_fp32_takes_no_low_order_part():
    q, k, v = qkv(torch.float32)
    with pytest.raises(ValueError):
        api.forward_train(q, k, v, o_lo_out=torch.empty_like(q))
    with pytest.raises(LibCalled):  # fp32: no o_lo, the call goes through
        api.forward_train(q, k, v)


def test_backward_rejects_malformed_buffers():
    q, k, v = qkv()
    o, lse, do = torch.zeros_like(q), torch.zeros(B, H, N), torch.zeros_like(q)
    need = 8 * B * H * N
    for ws in (torch.empty(need - 1, dtype=torch.uint8),            # too small
               torch.empty(need, dtype=torch.float32),               # not bytes
               torch.empty(2 * need, dtype=torch.uint8)[::2],        # not contiguous
               torch.empty(need, 2, dtype=torch.uint8),              # not 1-d
               bytearray(need)):                                     # not a tensor
        with pytest.raises(ValueError):
            api.backward(q, k, v, o, lse, do, workspace=ws)
    for name, bad in bad_outputs():
        with pytest.raises(ValueError):
            api.backward(q, k, v, o, lse, do, o_lo=bad)
    with pytest.raises(ValueError):  # o_lo with fp32 inputs
        qf, kf, vf = qkv(torch.float32)
        api.backward(qf, kf, vf, torch.zeros_like(qf), lse, torch.zeros_like(qf), o_lo=torch.zeros_like(qf))
    with pytest.raises(ValueError):
        api.backward(q, k, v, o[:, :, :-1], lse, do)
    with pytest.raises(ValueError):
        api.backward(q, k, v, o, lse[:, :, :-1], do)


def test_grouped_query_workspace_must_hold_the_partials():
    q, k, v = qkv(heads_kv=1)
    o, lse, do = torch.zeros_like(q), torch.zeros(B, H, N), torch.zeros_like(q)
    dense_need = 8 * B * H * N
    with pytest.raises(ValueError):
        api.backward(q, k, v, o, lse, do, workspace=torch.empty(dense_need, dtype=torch.uint8))
    gqa_need = FakeLib().fa_bwd_gqa_workspace_size(B, H, 1, N, D, 0)
    with pytest.raises(LibCalled):
        api.backward(q, k, v, o, lse, do, workspace=torch.empty(gqa_need, dtype=torch.uint8))


def test_grouped_query_shapes_never_reach_the_dense_entry_points():
    """K and V with H_kv < H heads hold B*H_kv*N*d elements; the dense fa_fwd / fa_bwd read
    B*H*N*d of each and would run past them.  The binding sends such shapes to the _gqa entry
    points, and refuses a head count that does not divide H, before any library call."""
    q, k, v = qkv(heads_kv=1)
    o, lse, do = torch.zeros_like(q), torch.zeros(B, H, N), torch.zeros_like(q)
    with pytest.raises(LibCalled, match="^fa_fwd_gqa$"):
        api.forward(q, k, v)
    mask = torch.ones(1, 1, dtype=torch.uint8)
    with pytest.raises(LibCalled, match="^fa_fwd_blocksparse_gqa$"):
        api.forward_blocksparse(q, k, v, mask)
    with pytest.raises(LibCalled, match="^fa_bwd_gqa$"):
        api.backward(q, k, v, o, lse, do)
    with pytest.raises(LibCalled, match="^fa_bwd_blocksparse_gqa$"):
        api.backward(q, k, v, o, lse, do, block_mask=mask)
    q3 = torch.zeros(B, 3, N, D, dtype=BF)
    k2, v2 = torch.zeros(B, 2, N, D, dtype=BF), torch.zeros(B, 2, N, D, dtype=BF)
    with pytest.raises(ValueError):
        api.forward(q3, k2, v2)
    with pytest.raises(ValueError):
        api.backward(q3, k2, v2, torch.zeros_like(q3), torch.zeros(B, 3, N), torch.zeros_like(q3))
