"""Seeded synthetic inputs for the exact-attention workloads.

This module is shared by the tests and the benchmark.  It holds no attention
arithmetic: only random draws, rounding of those draws to bfloat16, 128x128
tile masks and row samples.  Both the HIP path and the fp64 checker consume
the values it returns (the checker upcasts them exactly to float64).

The workload shapes stand in for the sequence lengths and head shapes that
the FlashAttention abstract (Tri Dao's author page on scite.ai) reports
results for: BERT-large at sequence length 512, GPT-2 at 1K, Path-X at 16K
and Path-256 at 64K.  Their datasets and weights are not used; iid Gaussian
activations of the same shapes replace them.  The grouped-query workload (the
FlashAttention-2 variants of the everydayai.blog article) uses the head counts
of a common 8B decoder, 32 query heads sharing 8 K/V heads, at 16K tokens.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np

SEED_ROOT = 35
# tensor slots inside a workload's seed sequence
SLOT_Q, SLOT_K, SLOT_V, SLOT_DO, SLOT_MASK, SLOT_ROWS = range(6)

MASK_BLOCK = 128  # granularity of the block-sparse tile mask (rows and keys)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int  # seed index of the workload (1..5)
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    qk_mult: float = 1.0  # multiplier applied to the Q and K draws
    sparse: bool = False
    density: float = 0.0  # fraction of strictly-lower off-diagonal tiles kept
    sample_rows: Optional[int] = None  # rows per head the checker evaluates
    backward: bool = False
    Hkv: Optional[int] = None  # K/V heads (grouped-query); None: as many as query heads

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.H, self.N, self.d)

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def kv_shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.kv_heads, self.N, self.d)

    @property
    def scale(self) -> float:
        # 1/sqrt(d) evaluated in fp32 and passed on as that fp32 value
        return float(np.float32(1.0) / np.sqrt(np.float32(self.d)))


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_f32", 1, 1, 1, 128, 64, "f32", False),
        Workload("bert_large_s512", 2, 8, 16, 512, 64, "bf16", False),
        Workload("gpt2_small_s1k", 3, 8, 12, 1024, 64, "bf16", True, backward=True),
        Workload("long_s16k_d128", 4, 1, 16, 16384, 128, "bf16", True, qk_mult=1.7, sample_rows=512),
        Workload("blocksparse_s64k", 5, 2, 16, 65536, 64, "bf16", True, sparse=True,
                 density=1.0 / 16.0, sample_rows=256),
        Workload("gqa_s16k_h32_kv8_d128", 6, 1, 32, 16384, 128, "bf16", True, sample_rows=256, Hkv=8),
    )
}


def rng_for(index: int, slot: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, index, slot]))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Works on the bit pattern: add 0x7FFF plus the lowest kept bit, then clear the
    low 16 bits.  NaN stays NaN (quiet), infinities stay infinities, and finite
    values past the largest bfloat16 round to infinity as IEEE rounding does.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    out = rounded.astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, (x.view(np.uint32) & 0xFFFF0000) | 0x00400000, out).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def draw(index: int, slot: int, shape: Sequence[int], mult: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """iid N(0,1) float32 draw times `mult`, rounded to bf16 unless dtype is f32."""
    x = rng_for(index, slot).standard_normal(tuple(shape), dtype=np.float32)
    if mult != 1.0:
        x = (x * np.float32(mult)).astype(np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    return x


def make_qkv(w: Workload, shape: Optional[Sequence[int]] = None):
    """Q, K, V (and dO when the workload has a backward) as float32 arrays.

    `shape` overrides the query shape [B, H, N, d]; K and V then keep the
    workload's query-to-K/V head ratio (at least one K/V head).
    """
    shape = tuple(shape) if shape is not None else w.shape
    kv = (shape[0], max(1, shape[1] * w.kv_heads // w.H), shape[2], shape[3])
    q = draw(w.index, SLOT_Q, shape, w.qk_mult, w.dtype)
    k = draw(w.index, SLOT_K, kv, w.qk_mult, w.dtype)
    v = draw(w.index, SLOT_V, kv, 1.0, w.dtype)
    do = draw(w.index, SLOT_DO, shape, 1.0, w.dtype) if w.backward else None
    return q, k, v, do


def make_block_mask(nb: int, density: float, seed_index: int, causal: bool = True) -> np.ndarray:
    """uint8 [nb, nb] tile mask: diagonal tiles on, plus an exact count of random off-diagonal tiles.

    The count is round(T * density) tiles drawn uniformly without replacement among
    the T candidate tiles: the strictly-lower ones when causal, else every
    off-diagonal tile.  An exact count makes the realised density deterministic.
    """
    mask = np.zeros((nb, nb), dtype=np.uint8)
    np.fill_diagonal(mask, 1)
    if causal:
        ii, jj = np.tril_indices(nb, k=-1)
    else:
        ii, jj = np.nonzero(~np.eye(nb, dtype=bool))
    T = ii.size
    count = int(round(T * density))
    if count > 0:
        pick = rng_for(seed_index, SLOT_MASK).choice(T, size=count, replace=False)
        mask[ii[pick], jj[pick]] = 1
    return mask


def sample_rows(N: int, count: int, seed_index: int, head: int = 0) -> np.ndarray:
    """Sorted query rows: the boundary rows {0, 1, 127, 128, N/2, N-1} plus uniform random others."""
    forced = sorted({r for r in (0, 1, 127, 128, N // 2, N - 1) if 0 <= r < N})
    count = min(count, N)
    rest = np.setdiff1d(np.arange(N), np.asarray(forced))
    rng = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, seed_index, SLOT_ROWS, head]))
    extra = rng.choice(rest, size=max(0, count - len(forced)), replace=False) if rest.size else []
    return np.sort(np.concatenate([np.asarray(forced, dtype=np.int64), np.asarray(extra, dtype=np.int64)]))


def random_case(seed: int, B: int, H: int, N: int, d: int, dtype: str = "bf16", mult: float = 1.0,
                backward: bool = False, h_kv: Optional[int] = None):
    """Small seeded case for edge tests (shapes outside the named workloads).

    Q and K are N(0,1) * mult, V (and dO) N(0,1), all rounded to bf16 unless dtype is f32.
    With h_kv, K and V are [B, h_kv, N, d] (grouped-query).
    """
    key = [SEED_ROOT, 100, seed, B, H, N, d] + ([] if h_kv is None else [h_kv])
    rng = np.random.default_rng(np.random.SeedSequence(key))
    out = []
    for t in range(4 if backward else 3):
        heads = h_kv if (h_kv is not None and t in (1, 2)) else H
        x = rng.standard_normal((B, heads, N, d), dtype=np.float32)
        if mult != 1.0 and t < 2:  # the multiplier scales Q and K only, as in the named workloads
            x = (x * np.float32(mult)).astype(np.float32)
        out.append(bf16_round(x) if dtype == "bf16" else x)
    if not backward:
        out.append(None)
    return tuple(out)


def random_block_mask(seed: int, nb: int, density: float, causal: bool) -> np.ndarray:
    """Seeded tile mask for edge tests; the diagonal is on, off-diagonal tiles are Bernoulli(density)."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 200, seed, nb]))
    mask = (rng.random((nb, nb)) < density).astype(np.uint8)
    np.fill_diagonal(mask, 1)
    if causal:
        mask = np.tril(mask)
    return mask


SLOT_SIGNS = 6  # random signs of the fp8 rotation


def random_signs(d: int, seed_index: int) -> np.ndarray:
    """int8 [d] of +-1: the random signs of the randomised Hadamard rotation (incoherent processing)."""
    rng = rng_for(seed_index, SLOT_SIGNS)
    return np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
