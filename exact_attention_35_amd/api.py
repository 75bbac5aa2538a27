"""Python binding of libfa: argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  Tensors are [B, H, N, d],
contiguous, on one GPU, bfloat16 or float32.  K and V may carry H_kv < H heads
(grouped-query; H_kv = 1 is multi-query): query head h then reads K/V head
h // (H // H_kv), and the dense entry points route to fa_fwd_gqa / fa_bwd_gqa.
"""

from __future__ import annotations

import contextlib
import functools
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.FA_F32, torch.bfloat16: _lib.FA_BF16}


def _on_gpu(t: torch.Tensor) -> bool:
    return t.is_cuda


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, allow_gqa: bool = False):
    """(B, H, N, d) of q, plus checks; with allow_gqa, k and v may be [B, H_kv, N, d], H_kv | H."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, N, d = q.shape
    hkv = k.shape[1]
    gqa_ok = allow_gqa and hkv >= 1 and H % hkv == 0
    if v.shape != k.shape or k.shape != (B, hkv if gqa_ok else H, N, d):
        raise ValueError(f"q, k, v shapes do not fit: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bfloat16 or float32")
    for t in (q, k, v):
        if not _on_gpu(t) or t.device != q.device:
            raise ValueError("q, k, v must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    return q.shape


def _check_buffer(t: torch.Tensor, shape, dtype: torch.dtype, device: torch.device, name: str) -> None:
    """A caller-supplied buffer must be exactly what the kernels will address: they write or
    read every element of `shape` in `dtype`, so anything else would be accessed out of bounds."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}; "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _outputs(q: torch.Tensor, out, lse_out, with_lse: bool):
    """o (caller's `out` or new) and lse (caller's `lse_out`, new, or None), checked."""
    B, H, N, _ = q.shape
    if out is None:
        o = torch.empty_like(q)
    else:
        _check_buffer(out, q.shape, q.dtype, q.device, "out")
        o = out
    lse = None
    if with_lse:
        if lse_out is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        else:
            _check_buffer(lse_out, (B, H, N), torch.float32, q.device, "lse_out")
            lse = lse_out
    elif lse_out is not None:
        raise ValueError("lse_out given with with_lse=False")
    return o, lse


@functools.lru_cache(maxsize=None)
def default_scale(d: int) -> float:
    """1/sqrt(d) as the fp32 value the kernels receive."""
    return float(torch.tensor(1.0, dtype=torch.float32) / torch.tensor(float(d), dtype=torch.float32).sqrt())


def _on_device(device: torch.device):
    """Make `device` current for the library call (a no-op when it already is)."""
    if device.index is None or torch.cuda.current_device() == device.index:
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
            causal: bool = False, with_lse: bool = True,
            out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact attention forward: returns (o, lse), lse fp32 [B, H, N] (None if with_lse=False).

    k and v may hold fewer heads than q (grouped-/multi-query, fa_fwd_gqa).
    """
    B, H, N, d = _check_qkv(q, k, v, allow_gqa=True)
    hkv = k.shape[1]
    scale = default_scale(d) if scale is None else float(scale)
    o, lse = _outputs(q, out, lse_out, with_lse)
    lib = _lib.load()
    lse_ptr = lse.data_ptr() if lse is not None else None
    with _on_device(q.device):
        if hkv == H:
            st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_ptr, B, H, N, d, scale,
                            int(bool(causal)), _DTYPES[q.dtype], _stream_ptr(q.device))
        else:
            st = lib.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_ptr, B, H, hkv, N, d,
                                scale, int(bool(causal)), _DTYPES[q.dtype], _stream_ptr(q.device))
    _lib.check(st, "fa_fwd" if hkv == H else "fa_fwd_gqa")
    return o, lse


def forward_blocksparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: torch.Tensor,
                        scale: Optional[float] = None, causal: bool = False, with_lse: bool = True,
                        out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Block-sparse forward; block_mask is uint8 [ceil(N/128), ceil(N/128)] on the same GPU.

    k and v may hold fewer heads than q (grouped-/multi-query, fa_fwd_blocksparse_gqa).
    """
    B, H, N, d = _check_qkv(q, k, v, allow_gqa=True)
    hkv = k.shape[1]
    _check_mask(block_mask, N, q.device)
    scale = default_scale(d) if scale is None else float(scale)
    o, lse = _outputs(q, out, lse_out, with_lse)
    lib = _lib.load()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), block_mask.data_ptr(), o.data_ptr(),
            lse.data_ptr() if lse is not None else None)
    tail = (N, d, scale, int(bool(causal)), _DTYPES[q.dtype], _stream_ptr(q.device))
    with _on_device(q.device):
        if hkv == H:
            st = lib.fa_fwd_blocksparse(*ptrs, B, H, *tail)
        else:
            st = lib.fa_fwd_blocksparse_gqa(*ptrs, B, H, hkv, *tail)
    _lib.check(st, "fa_fwd_blocksparse" if hkv == H else "fa_fwd_blocksparse_gqa")
    return o, lse


def forward_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                  causal: bool = False, block_mask: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                  o_lo_out: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Forward for training (fa_fwd_ex): (o, lse, o_lo).

    For bf16 inputs o_lo is the low-order bf16 part of the output (o + o_lo carries the fp32
    result); hand it to backward(..., o_lo=o_lo) so that D = rowsum(dO * O) is formed from it.
    For fp32 inputs o_lo is None.  block_mask and grouped-query K/V as for forward_blocksparse.
    """
    B, H, N, d = _check_qkv(q, k, v, allow_gqa=True)
    hkv = k.shape[1]
    if block_mask is not None:
        _check_mask(block_mask, N, q.device)
    scale = default_scale(d) if scale is None else float(scale)
    o, lse = _outputs(q, out, lse_out, True)
    o_lo = None
    if q.dtype == torch.bfloat16:
        if o_lo_out is None:
            o_lo = torch.empty_like(q)
        else:
            _check_buffer(o_lo_out, q.shape, q.dtype, q.device, "o_lo_out")
            o_lo = o_lo_out
    elif o_lo_out is not None:
        raise ValueError("o_lo_out applies to bfloat16 inputs only")
    lib = _lib.load()
    with _on_device(q.device):
        st = lib.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           None if block_mask is None else block_mask.data_ptr(), o.data_ptr(),
                           None if o_lo is None else o_lo.data_ptr(), lse.data_ptr(), B, H, hkv, N, d, scale,
                           int(bool(causal)), _DTYPES[q.dtype], _stream_ptr(q.device))
    _lib.check(st, "fa_fwd_ex")
    return o, lse, o_lo


def bwd_workspace_size(B: int, H: int, N: int, d: int, grad_dtype: torch.dtype = torch.float32,
                       H_kv: Optional[int] = None) -> int:
    if H_kv is None or H_kv == H:
        return int(_lib.load().fa_bwd_workspace_size(B, H, N, d, _DTYPES[grad_dtype]))
    return int(_lib.load().fa_bwd_gqa_workspace_size(B, H, H_kv, N, d, _DTYPES[grad_dtype]))


def _check_mask(block_mask: torch.Tensor, N: int, device: torch.device) -> None:
    nb = -(-N // _lib.FA_MASK_BLOCK)
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be uint8 [{nb}, {nb}]")
    if not block_mask.is_contiguous() or block_mask.device != device:
        raise ValueError("block_mask must be contiguous and on the same GPU as q")


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             do: torch.Tensor, scale: Optional[float] = None, causal: bool = False,
             grad_dtype: torch.dtype = torch.float32, workspace: Optional[torch.Tensor] = None,
             block_mask: Optional[torch.Tensor] = None, o_lo: Optional[torch.Tensor] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dq, dk, dv) of sum(do * o), in grad_dtype (float32 by default).

    With block_mask (uint8 [ceil(N/128), ceil(N/128)], as for forward_blocksparse) this is
    the block-sparse backward, fa_bwd_blocksparse.  With k and v of H_kv < H heads it is the
    grouped-query backward, fa_bwd_gqa (with a mask too: fa_bwd_blocksparse_gqa); dk and dv
    then have k's shape.  With o_lo (from forward_train) the call is fa_bwd_ex, which forms
    D = rowsum(do * O) from o + o_lo.  `workspace`, if given, is a contiguous uint8 tensor on
    q's device of at least bwd_workspace_size(...) bytes.
    """
    B, H, N, d = _check_qkv(q, k, v, allow_gqa=True)
    hkv = k.shape[1]
    if block_mask is not None:
        _check_mask(block_mask, N, q.device)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device, and be contiguous")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be contiguous float32 [B, H, N] on q's device")
    if o_lo is not None:
        if q.dtype != torch.bfloat16:
            raise ValueError("o_lo applies to bfloat16 inputs only")
        _check_buffer(o_lo, q.shape, q.dtype, q.device, "o_lo")
    if grad_dtype not in _DTYPES:
        raise ValueError("grad_dtype must be torch.float32 or torch.bfloat16")
    scale = default_scale(d) if scale is None else float(scale)
    dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    dv = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    need = bwd_workspace_size(B, H, N, d, grad_dtype, hkv)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or workspace.dim() != 1
          or not workspace.is_contiguous() or workspace.device != q.device or workspace.numel() < need):
        raise ValueError(f"workspace must be a contiguous 1-d uint8 tensor of at least {need} bytes on {q.device}")
    lib = _lib.load()
    tail = (N, d, scale, int(bool(causal)), _DTYPES[q.dtype], _DTYPES[grad_dtype], workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_ptr(q.device))
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    with _on_device(q.device):
        if o_lo is not None:
            name = "fa_bwd_ex"
            st = lib.fa_bwd_ex(*ptrs[:3], None if block_mask is None else block_mask.data_ptr(), ptrs[3],
                               o_lo.data_ptr(), *ptrs[4:], B, H, hkv, *tail)
        elif block_mask is not None and hkv == H:
            name = "fa_bwd_blocksparse"
            st = lib.fa_bwd_blocksparse(*ptrs[:3], block_mask.data_ptr(), *ptrs[3:], B, H, *tail)
        elif block_mask is not None:
            name = "fa_bwd_blocksparse_gqa"
            st = lib.fa_bwd_blocksparse_gqa(*ptrs[:3], block_mask.data_ptr(), *ptrs[3:], B, H, hkv, *tail)
        elif hkv != H:
            name = "fa_bwd_gqa"
            st = lib.fa_bwd_gqa(*ptrs, B, H, hkv, *tail)
        else:
            name = "fa_bwd"
            st = lib.fa_bwd(*ptrs, B, H, *tail)
    _lib.check(st, name)
    return dq, dk, dv


def backward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                     do: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                     scale: Optional[float] = None, causal: bool = False, block_mask: Optional[torch.Tensor] = None,
                     o_lo: Optional[torch.Tensor] = None) -> None:
    """fa_bwd_noalloc: the backward into caller-given dq, dk, dv (fp32 or bf16, all one dtype)
    with the library's static device workspace instead of a caller workspace; nothing is
    allocated, so it may be captured in a HIP graph.  Calls that overlap on one GPU race on
    that workspace.  Arguments otherwise as backward()."""
    B, H, N, d = _check_qkv(q, k, v, allow_gqa=True)
    hkv = k.shape[1]
    if block_mask is not None:
        _check_mask(block_mask, N, q.device)
    for name, t in (("o", o), ("do", do)):
        _check_buffer(t, q.shape, q.dtype, q.device, name)
    _check_buffer(lse, (B, H, N), torch.float32, q.device, "lse")
    if o_lo is not None:
        if q.dtype != torch.bfloat16:
            raise ValueError("o_lo applies to bfloat16 inputs only")
        _check_buffer(o_lo, q.shape, q.dtype, q.device, "o_lo")
    grad_dtype = dq.dtype if isinstance(dq, torch.Tensor) else None
    if grad_dtype not in _DTYPES:
        raise ValueError("dq must be a float32 or bfloat16 tensor")
    _check_buffer(dq, q.shape, grad_dtype, q.device, "dq")
    _check_buffer(dk, k.shape, grad_dtype, q.device, "dk")
    _check_buffer(dv, k.shape, grad_dtype, q.device, "dv")
    scale = default_scale(d) if scale is None else float(scale)
    lib = _lib.load()
    with _on_device(q.device):
        st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                None if block_mask is None else block_mask.data_ptr(), o.data_ptr(),
                                None if o_lo is None else o_lo.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, hkv, N, d, scale,
                                int(bool(causal)), _DTYPES[q.dtype], _DTYPES[grad_dtype], _stream_ptr(q.device))
    _lib.check(st, "fa_bwd_noalloc")


class FlashAttentionFunction(torch.autograd.Function):
    """autograd wrapper: forward (fa_fwd_ex) saves q, k, v, o, lse, the low-order part of o
    (bf16 inputs) and the block mask; backward calls fa_bwd_ex with them (fp32 inputs: fa_bwd
    and its variants)."""

    @staticmethod
    def forward(ctx, q, k, v, scale=None, causal=False, block_mask=None):
        o, lse, o_lo = forward_train(q, k, v, scale, causal, block_mask)
        ctx.save_for_backward(q, k, v, o, lse, o_lo, block_mask)
        ctx.scale = default_scale(q.shape[-1]) if scale is None else float(scale)
        ctx.causal = causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, o_lo, mask = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), ctx.scale, ctx.causal, grad_dtype=q.dtype,
                              block_mask=mask, o_lo=o_lo)
        return dq, dk, dv, None, None, None


def attention(q, k, v, scale=None, causal=False, block_mask=None):
    """Differentiable exact attention (bf16 gradients for bf16 inputs).

    k, v may have H_kv | H heads (grouped-/multi-query); block_mask (uint8
    [ceil(N/128), ceil(N/128)]) makes it block-sparse, with or without grouped heads.
    """
    return FlashAttentionFunction.apply(q, k, v, scale, causal, block_mask)


def fp8_scale_shape(B: int, H: int, N: int) -> Tuple[int, int, int]:
    """Shape of the per-block fp8 scales: [B, H, ceil(N / 128)]."""
    return (B, H, -(-N // _lib.FA_FP8_BLOCK))


def quantize_fp8(x: torch.Tensor, signs: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(codes uint8 [B, H, N, d], scales float32 [B, H, ceil(N/128)]) of x (bf16 or fp32, [B, H, N, d]).

    signs: optional int8 [d] of +-1 on x's device; the rows are then rotated by the
    randomised Hadamard transform first (incoherent processing; use the same signs
    for Q and K and none for V).
    """
    if x.dim() != 4 or x.dtype not in _DTYPES or not _on_gpu(x) or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, N, d] bf16 or float32 GPU tensor")
    B, H, N, d = x.shape
    if signs is not None:
        if signs.dtype != torch.int8 or tuple(signs.shape) != (d,) or signs.device != x.device:
            raise ValueError(f"signs must be int8 [{d}] on x's device")
        signs = signs.contiguous()
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty(fp8_scale_shape(B, H, N), dtype=torch.float32, device=x.device)
    with _on_device(x.device):
        st = _lib.load().fa_quantize_fp8(x.data_ptr(), None if signs is None else signs.data_ptr(),
                                         codes.data_ptr(), scales.data_ptr(), B, H, N, d, _DTYPES[x.dtype],
                                         _stream_ptr(x.device))
    _lib.check(st, "fa_quantize_fp8")
    return codes, scales


def forward_fp8(q8: torch.Tensor, q_scale: torch.Tensor, k8: torch.Tensor, k_scale: torch.Tensor,
                v8: torch.Tensor, v_scale: torch.Tensor, scale: Optional[float] = None, causal: bool = False,
                with_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """FP8 forward on quantize_fp8 outputs: (o bf16 [B, H, N, d], lse fp32 [B, H, N] or None).

    k8, v8 may have H_kv | H heads (grouped-query).
    """
    for t in (q8, k8, v8):
        if t.dim() != 4 or t.dtype != torch.uint8 or not _on_gpu(t) or not t.is_contiguous() or t.device != q8.device:
            raise ValueError("q8, k8, v8 must be contiguous uint8 [B, H, N, d] tensors on one GPU")
    B, H, N, d = q8.shape
    hkv = k8.shape[1]
    if v8.shape != k8.shape or k8.shape != (B, hkv, N, d) or hkv < 1 or H % hkv:
        raise ValueError(f"q8, k8, v8 shapes do not fit: {tuple(q8.shape)} {tuple(k8.shape)} {tuple(v8.shape)}")
    for name, t, heads in (("q_scale", q_scale, H), ("k_scale", k_scale, hkv), ("v_scale", v_scale, hkv)):
        if (tuple(t.shape) != fp8_scale_shape(B, heads, N) or t.dtype != torch.float32 or not t.is_contiguous()
                or t.device != q8.device):
            raise ValueError(f"{name} must be contiguous float32 {fp8_scale_shape(B, heads, N)} on q8's device")
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if with_lse else None
    with _on_device(q8.device):
        st = _lib.load().fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_scale.data_ptr(),
                                    k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(),
                                    None if lse is None else lse.data_ptr(), B, H, hkv, N, d, scale,
                                    int(bool(causal)), _stream_ptr(q8.device))
    _lib.check(st, "fa_fwd_fp8")
    return o, lse
