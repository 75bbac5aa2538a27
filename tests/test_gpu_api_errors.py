"""The Python binding rejects malformed arguments with ValueError before calling the library,
and the library's own status codes surface as FaError."""

import pytest
import torch

from exact_attention_35_amd import _lib, api

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF = torch.bfloat16


def _t(shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def test_forward_argument_errors():
    q = _t((1, 4, 64, 64))
    with pytest.raises(ValueError):
        api.forward(q, _t((1, 4, 64, 128)), _t((1, 4, 64, 128)))          # head dims differ
    with pytest.raises(ValueError):
        api.forward(q, _t((1, 3, 64, 64)), _t((1, 3, 64, 64)))            # 3 K/V heads for 4 query heads
    with pytest.raises(ValueError):
        api.forward(q, _t((1, 4, 64, 64), torch.float32), _t((1, 4, 64, 64)))  # dtype mismatch
    with pytest.raises(ValueError):
        api.forward(q, _t((1, 4, 64, 64)).transpose(2, 3), _t((1, 4, 64, 64)))  # not contiguous
    with pytest.raises(ValueError):
        api.forward(q.cpu(), q.cpu(), q.cpu())                            # not on the GPU
    with pytest.raises(ValueError):
        api.forward(q, q, q[..., :32].contiguous())                       # V shape differs


def test_library_status_surfaces():
    q = _t((1, 2, 64, 96))  # d = 96: the library reports FA_ERR_UNSUPPORTED
    with pytest.raises(_lib.FaError) as e:
        api.forward(q, q, q)
    assert e.value.status == _lib.FA_ERR_UNSUPPORTED


def test_backward_and_sparse_argument_errors():
    q = _t((1, 2, 200, 64))
    o, lse = api.forward(q, q, q)
    with pytest.raises(ValueError):
        api.backward(q, q, q, o, lse[:, :, :100].contiguous(), q)         # lse shape
    with pytest.raises(ValueError):
        api.backward(q, q, q, o.float(), lse, q)                          # o dtype
    with pytest.raises(ValueError):
        api.forward_blocksparse(q, q, q, torch.ones((1, 1), dtype=torch.uint8, device=DEV))  # mask shape
    with pytest.raises(ValueError):
        api.backward(q, q, q, o, lse, q, block_mask=torch.ones((2, 2), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()


def test_fp8_argument_errors():
    x = _t((1, 2, 200, 64))
    with pytest.raises(ValueError):
        api.quantize_fp8(x, torch.ones(32, dtype=torch.int8, device=DEV))  # signs of the wrong length
    with pytest.raises(ValueError):
        api.quantize_fp8(x.half())                                        # fp16 input
    c, s = api.quantize_fp8(x)
    with pytest.raises(ValueError):
        api.forward_fp8(c, s[:, :, :1].contiguous(), c, s, c, s)          # scale shape
    with pytest.raises(ValueError):
        api.forward_fp8(c, s, c[:, :1].contiguous(), s, c, s)             # K heads without matching scales
    torch.cuda.synchronize()
