"""Python binding of libfa: argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  Tensors are [B, H, N, d],
contiguous, on one GPU, bfloat16 or float32.
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.FA_F32, torch.bfloat16: _lib.FA_BF16}


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bfloat16 or float32")
    for t in (q, k, v):
        if not t.is_cuda or t.device != q.device:
            raise ValueError("q, k, v must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    return q.shape


def default_scale(d: int) -> float:
    """1/sqrt(d) as the fp32 value the kernels receive."""
    return float(torch.tensor(1.0, dtype=torch.float32) / torch.tensor(float(d), dtype=torch.float32).sqrt())


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
            causal: bool = False, with_lse: bool = True,
            out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact attention forward: returns (o, lse), lse fp32 [B, H, N] (None if with_lse=False)."""
    B, H, N, d = _check_qkv(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = None
    if with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse_out is None else lse_out
    with torch.cuda.device(q.device):
        st = _lib.load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, H, N, d, scale,
                                int(bool(causal)), _DTYPES[q.dtype], _stream_ptr(q.device))
    _lib.check(st, "fa_fwd")
    return o, lse


def forward_blocksparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: torch.Tensor,
                        scale: Optional[float] = None, causal: bool = False, with_lse: bool = True,
                        out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Block-sparse forward; block_mask is uint8 [ceil(N/128), ceil(N/128)] on the same GPU."""
    B, H, N, d = _check_qkv(q, k, v)
    nb = -(-N // _lib.FA_MASK_BLOCK)
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be uint8 [{nb}, {nb}]")
    if not block_mask.is_contiguous() or block_mask.device != q.device:
        raise ValueError("block_mask must be contiguous and on the same GPU as q")
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = None
    if with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse_out is None else lse_out
    with torch.cuda.device(q.device):
        st = _lib.load().fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), block_mask.data_ptr(),
                                            o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                            B, H, N, d, scale, int(bool(causal)), _DTYPES[q.dtype],
                                            _stream_ptr(q.device))
    _lib.check(st, "fa_fwd_blocksparse")
    return o, lse


def bwd_workspace_size(B: int, H: int, N: int, d: int, grad_dtype: torch.dtype = torch.float32) -> int:
    return int(_lib.load().fa_bwd_workspace_size(B, H, N, d, _DTYPES[grad_dtype]))


def _check_mask(block_mask: torch.Tensor, N: int, device: torch.device) -> None:
    nb = -(-N // _lib.FA_MASK_BLOCK)
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be uint8 [{nb}, {nb}]")
    if not block_mask.is_contiguous() or block_mask.device != device:
        raise ValueError("block_mask must be contiguous and on the same GPU as q")


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             do: torch.Tensor, scale: Optional[float] = None, causal: bool = False,
             grad_dtype: torch.dtype = torch.float32, workspace: Optional[torch.Tensor] = None,
             block_mask: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dq, dk, dv) of sum(do * o), in grad_dtype (float32 by default).

    With block_mask (uint8 [ceil(N/128), ceil(N/128)], as for forward_blocksparse) this is
    the block-sparse backward, fa_bwd_blocksparse.
    """
    B, H, N, d = _check_qkv(q, k, v)
    if block_mask is not None:
        _check_mask(block_mask, N, q.device)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device, and be contiguous")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be contiguous float32 [B, H, N] on q's device")
    if grad_dtype not in _DTYPES:
        raise ValueError("grad_dtype must be torch.float32 or torch.bfloat16")
    scale = default_scale(d) if scale is None else float(scale)
    dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    dk = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    dv = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    need = bwd_workspace_size(B, H, N, d, grad_dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    lib = _lib.load()
    tail = (B, H, N, d, scale, int(bool(causal)), _DTYPES[q.dtype], _DTYPES[grad_dtype], workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_ptr(q.device))
    with torch.cuda.device(q.device):
        if block_mask is None:
            st = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *tail)
        else:
            st = lib.fa_bwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), block_mask.data_ptr(),
                                        o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                        dv.data_ptr(), *tail)
    _lib.check(st, "fa_bwd" if block_mask is None else "fa_bwd_blocksparse")
    return dq, dk, dv


class FlashAttentionFunction(torch.autograd.Function):
    """autograd wrapper: forward saves (q, k, v, o, lse); backward calls fa_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, scale=None, causal=False):
        o, lse = forward(q, k, v, scale, causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale = default_scale(q.shape[-1]) if scale is None else float(scale)
        ctx.causal = causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), ctx.scale, ctx.causal, grad_dtype=q.dtype)
        return dq, dk, dv, None, None


def attention(q, k, v, scale=None, causal=False):
    """Differentiable exact attention (bf16 gradients for bf16 inputs)."""
    return FlashAttentionFunction.apply(q, k, v, scale, causal)
