"""ctypes loader of libfa.so (the HIP kernels behind the C ABI of include/fa.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_HIP = -4
FA_ERR_SCRATCH = -5
FA_F32 = 0
FA_BF16 = 1
FA_MASK_BLOCK = 128
FA_FP8_BLOCK = 128
FA_NOALLOC_SCRATCH_BYTES = 32 << 20
FA_ABI_VERSION = 5  # must equal FA_ABI_VERSION of include/fa.h

EXPORTS = ("fa_fwd", "fa_fwd_gqa", "fa_fwd_blocksparse", "fa_bwd_workspace_size", "fa_bwd",
           "fa_bwd_gqa_workspace_size", "fa_bwd_gqa", "fa_bwd_blocksparse", "fa_fwd_blocksparse_gqa",
           "fa_bwd_blocksparse_gqa", "fa_fwd_ex", "fa_bwd_ex", "fa_bwd_noalloc", "fa_quantize_fp8", "fa_fwd_fp8",
           "fa_status_string", "fa_version")

_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


class FaError(RuntimeError):
    """A libfa entry point returned a negative status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    # Bind to the HIP runtime that torch (which owns the memory and streams we are
    # given) has loaded: loading libfa.so first would pull in a second runtime.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m exact_attention_35_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_version.restype = _i
    lib.fa_version.argtypes = []
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [_i]
    lib.fa_fwd.restype = _i
    lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_fwd_gqa.restype = _i
    lib.fa_fwd_gqa.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_fwd_blocksparse.restype = _i
    lib.fa_fwd_blocksparse.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_size.argtypes = [_i, _i, _i, _i, _i]
    lib.fa_bwd.restype = _i
    lib.fa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _i,
                           _vp, ctypes.c_size_t, _vp]
    lib.fa_bwd_gqa_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd_gqa_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
    lib.fa_bwd_gqa.restype = _i
    lib.fa_bwd_gqa.argtypes = [_vp] * 9 + [_i, _i, _i, _i, _i, _f, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.fa_quantize_fp8.restype = _i
    lib.fa_quantize_fp8.argtypes = [_vp] * 4 + [_i] * 5 + [_vp]
    lib.fa_fwd_fp8.restype = _i
    lib.fa_fwd_fp8.argtypes = [_vp] * 8 + [_i] * 5 + [_f, _i, _vp]
    lib.fa_bwd_blocksparse.restype = _i
    lib.fa_bwd_blocksparse.argtypes = [_vp] * 10 + [_i, _i, _i, _i, _f, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.fa_fwd_blocksparse_gqa.restype = _i
    lib.fa_fwd_blocksparse_gqa.argtypes = [_vp] * 6 + [_i, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_bwd_blocksparse_gqa.restype = _i
    lib.fa_bwd_blocksparse_gqa.argtypes = [_vp] * 10 + [_i, _i, _i, _i, _i, _f, _i, _i, _i, _vp, ctypes.c_size_t,
                                                        _vp]
    lib.fa_fwd_ex.restype = _i
    lib.fa_fwd_ex.argtypes = [_vp] * 7 + [_i] * 5 + [_f, _i, _i, _vp]
    lib.fa_bwd_ex.restype = _i
    lib.fa_bwd_ex.argtypes = [_vp] * 11 + [_i] * 5 + [_f, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
    lib.fa_bwd_noalloc.restype = _i
    lib.fa_bwd_noalloc.argtypes = [_vp] * 11 + [_i] * 5 + [_f, _i, _i, _i, _vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != FA_OK:
        raise FaError(status, what)
