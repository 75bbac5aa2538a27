// LDS tile machinery shared by the gfx950 attention kernels: tile layouts,
// LDS-direct tile loads, the MFMA passes over a tile, and barriers.
//
// A tile is BN rows (keys or queries) x D bf16 values of one head, row-major
// in HBM.  In LDS it is row-major with 16-byte chunks permuted by an XOR of the
// row ("swizzle") so that MFMA operand reads hit distinct LDS banks.
#pragma once

#include "fa_device.hpp"

namespace fa {

// Hide a per-lane offset from loop-invariant code motion: the addresses derived
// from it are then formed next to their use, instead of being kept live in VGPRs
// across a whole loop for every buffer of a ring.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int D, int BN>
struct TileCfg {
  static constexpr int NC = D / 8;          // 16-byte chunks per row
  static constexpr int RPK = 64 / NC;       // rows written by one 1 KB LDS-direct load
  static constexpr int TILE = BN * D;       // elements of one tile
  static constexpr int NSB = BN / 32;       // 32-row MFMA blocks per tile
  static constexpr int NPT = BN / 16;       // 16-row bf16 fragments per tile
  static constexpr int KB_PER_WAVE = BN * D * 2 / 1024 / 4;  // 1 KB loads per wave when 4 waves load a tile
  static_assert(KB_PER_WAVE * 4 * 1024 == BN * D * 2, "a tile is a whole number of 1 KB loads per wave");
};

// ---- Two layouts:
//   K layout: row R holds row swap23(R) of the tile; chunk c sits at c ^ swz_k(R).
//      Row reads: 32 lanes x 16 B of one chunk column over 32 consecutive rows.
//   V layout: row R holds row R; chunk c sits at c ^ swz_v(R).  Read with the
//      transposing LDS read (4 rows x 16 columns per 16-lane group).
// K layout swizzle: a bijection on the 16 (d = 128) or 8 (d = 64, two rows per
// 256-byte bank line) rows of a bank group, so the 16 lanes of a 16-byte row
// read hit distinct banks; it also spreads any 4 consecutive rows x 4
// consecutive chunks over distinct banks, which the transposing reads need.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Tile kt -> LDS with 1 KB LDS-direct loads; NW waves (index wi) cover the tile
// together.  Rows past the end of the buffer resource read as zeros.
template <int D, int BN, int NW = 4>
__device__ __forceinline__ void dma_k(BufRes kres, unsigned short* kbuf, int kt, int wi, int lane) {
  using C = TileCfg<D, BN>;
  constexpr int LPW = BN * D * 2 / 1024 / NW;  // loads per wave
  static_assert(LPW * NW * 1024 == BN * D * 2, "a tile is a whole number of 1 KB loads per wave");
#pragma unroll
  for (int n = 0; n < LPW; ++n) {
    const int blk = wi * LPW + n;
    const int row = blk * C::RPK + lane / C::NC;
    const int c = (lane % C::NC) ^ swz_k<D>(row);
    const unsigned int off = (unsigned int)((kt * BN + swap23(row)) * D + c * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (lds_void_t*)(kbuf + blk * 512), 16, off, 0, 0, 0);
  }
}

template <int D, int BN, int NW = 4>
__device__ __forceinline__ void dma_v(BufRes vres, unsigned short* vbuf, int kt, int wi, int lane) {
  using C = TileCfg<D, BN>;
  constexpr int LPW = BN * D * 2 / 1024 / NW;
  static_assert(LPW * NW * 1024 == BN * D * 2, "a tile is a whole number of 1 KB loads per wave");
#pragma unroll
  for (int n = 0; n < LPW; ++n) {
    const int blk = wi * LPW + n;
    const int row = blk * C::RPK + lane / C::NC;
    const int c = (lane % C::NC) ^ swz_v<D>(row);
    const unsigned int off = (unsigned int)((kt * BN + row) * D + c * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (lds_void_t*)(vbuf + blk * 512), 16, off, 0, 0, 0);
  }
}

// Block-sparse schedules: one wave lists, in ascending order, the indices i in
// [first, end) whose mask flag flags[i * stride] is nonzero, into list[] in LDS, and
// returns their count (wave-uniform).  The flags of 512 indices are requested before
// any of them is examined, so the scan waits for one round of loads per 512 indices
// instead of one per 64.
__device__ __forceinline__ int list_kept(const unsigned char* flags, size_t stride, int first, int end,
                                         unsigned short* list, int lane) {
  int cnt = 0;
  for (int base = first; base < end; base += 512) {
    unsigned char f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // unconditional loads (indices past the end re-read the last flag)
      const int i = min(base + 64 * u + lane, end - 1);
      f[u] = flags[(size_t)i * stride];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + 64 * u + lane;
      const bool on = i < end && f[u] != 0;
      const unsigned long long bal = __ballot(on);
      if (on) list[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (unsigned short)i;
      cnt += __popcll(bal);
    }
  }
  return cnt;
}

// wait for this wave's LDS-direct loads (they count as vector-memory loads)
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// wait for all but the N most recent vector-memory loads (N < 16)
template <int N>
__device__ __forceinline__ void wait_dma_but() { __builtin_amdgcn_s_waitcnt(0x0F70 | N); }

// Per-lane element offsets of the S^T operand reads (one per 16-wide d chunk).
template <int D>
struct KOffsets {
  int off[D / 16];
};
template <int D>
__device__ __forceinline__ KOffsets<D> k_offsets(int l32, int half) {
  KOffsets<D> k;
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) k.off[cc] = l32 * D + (((2 * cc + half) ^ swz_k<D>(l32)) * 8);
  return k;
}

// ---- S^T = K Q^T for one key tile: lane (query l32, half h), register r of block b
// holds key 32b + 16(r/8) + 8h + (r%8) of the tile (K rows are swap23-ordered in LDS).
template <int D, int BN>
__device__ __forceinline__ void qk_tile(const unsigned short* kbuf, const KOffsets<D>& ko, const bf16x8 (&qf)[D / 16],
                                        f32x16 (&s)[TileCfg<D, BN>::NSB]) {
  using C = TileCfg<D, BN>;
#pragma unroll
  for (int b = 0; b < C::NSB; ++b) s[b] = zero16();
  int o[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) o[cc] = fresh(ko.off[cc]);
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
#pragma unroll
    for (int b = 0; b < C::NSB; ++b) s[b] = mfma32(lds_bf16x8(kbuf + 32 * b * D + o[cc]), qf[cc], s[b]);
  }
}

// Two row-read tile products at once, S += X1 F1 and P += X2 F2 (both tiles in the
// K layout, same shape), interleaved as four independent accumulator chains, with
// the LDS operands loaded PF MFMAs ahead into a register ring.
template <int D, int BN, int PF = 4>
__device__ __forceinline__ void qk_pair_tile(const unsigned short* buf1, const unsigned short* buf2,
                                             const KOffsets<D>& ko, const bf16x8 (&f1)[D / 16],
                                             const bf16x8 (&f2)[D / 16], f32x16 (&s1)[BN / 32],
                                             f32x16 (&s2)[BN / 32]) {
  constexpr int NSB = BN / 32;
  constexpr int NM = 2 * NSB * (D / 16);
  // MFMA m: chunk cc = m / (2 NSB), block b = (m / 2) % NSB, tile (m % 2)
  int o[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) o[cc] = fresh(ko.off[cc]);
  auto operand = [&](int m) __attribute__((always_inline)) -> bf16x8 {
    const int cc = m / (2 * NSB);
    const int b = (m >> 1) % NSB;
    return lds_bf16x8(((m & 1) ? buf2 : buf1) + 32 * b * D + o[cc]);
  };
#pragma unroll
  for (int b = 0; b < NSB; ++b) {
    s1[b] = zero16();
    s2[b] = zero16();
  }
  bf16x8 ring[PF];
#pragma unroll
  for (int m = 0; m < PF; ++m) ring[m] = operand(m);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const bf16x8 x = ring[m % PF];
    if (m + PF < NM) ring[m % PF] = operand(m + PF);
    const int cc = m / (2 * NSB);
    const int b = (m >> 1) % NSB;
    if (m & 1) s2[b] = mfma32(x, f2[cc], s2[b]);
    else s1[b] = mfma32(x, f1[cc], s1[b]);
  }
}

// One row-read tile product S += X F (tile in the K layout), its LDS operands loaded
// PF MFMAs ahead into a register ring.  S is not cleared: the caller sets its start.
template <int D, int BN, int PF = 4>
__device__ __forceinline__ void qk_ring_tile(const unsigned short* buf, const KOffsets<D>& ko,
                                             const bf16x8 (&f)[D / 16], f32x16 (&s)[BN / 32]) {
  constexpr int NSB = BN / 32;
  constexpr int NM = NSB * (D / 16);
  // MFMA m: chunk cc = m / NSB, block b = m % NSB
  int o[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) o[cc] = fresh(ko.off[cc]);
  auto operand = [&](int m) __attribute__((always_inline)) -> bf16x8 {
    return lds_bf16x8(buf + 32 * (m % NSB) * D + o[m / NSB]);
  };
  bf16x8 ring[PF];
#pragma unroll
  for (int m = 0; m < PF; ++m) ring[m] = operand(m);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const bf16x8 x = ring[m % PF];
    if (m + PF < NM) ring[m % PF] = operand(m + PF);
    s[m % NSB] = mfma32(x, f[m / NSB], s[m % NSB]);
  }
}

// Per-lane element offsets of the transposing V reads: base (row part) and one
// chunk offset per 32-wide d block.
template <int D>
struct VOffsets {
  int base;
  int blk[D / 32];
};
template <int D>
__device__ __forceinline__ VOffsets<D> v_offsets(int lane) {
  VOffsets<D> v;
  const int half = lane >> 5;
  const int g = lane >> 4;   // 16-lane group: (half, which 16 of the 32 d)
  const int j = lane & 15;   // source row (j/4) and 4-element column group (j%4)
  const int dsub = g & 1;
  const int row = 8 * half + (j >> 2);  // + 16t + 4r at the call
  v.base = row * D + (j & 1) * 4;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int c = 4 * db + 2 * dsub + ((j & 3) >> 1);
    v.blk[db] = (c ^ swz_v<D>(row)) * 8;
  }
  return v;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ uint2 lds_read_tr(const unsigned short* p) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((__attribute__((address_space(3))) unsigned short*)p));
  return __builtin_bit_cast(uint2, r);
}

// O^T += V^T P^T: lane (query l32, half h), d block db, register r holds d = 32db + 8(r/4) + 4h + r%4.
// The V^T operand (8 keys 16t + 8h + e for d = 32db + l32) comes from two transposing reads.
template <int D, int BN>
__device__ __forceinline__ void pv_tile(const unsigned short* vbuf, const VOffsets<D>& vo, const bf16x8 (&pf)[BN / 16],
                                        f32x16 (&oacc)[D / 32]) {
  int o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = fresh(vo.base + vo.blk[db]);
#pragma unroll
  for (int t = 0; t < BN / 16; ++t) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned short* p = vbuf + o[db] + 16 * t * D;
      const uint2 lo = lds_read_tr(p);
      const uint2 hi = lds_read_tr(p + 4 * D);
      oacc[db] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pf[t], oacc[db]);
    }
  }
}

// Per-lane element offsets of the transposing reads of a K-layout tile: for the
// 16-row chunk t, rows 16t + 8h + 4r + j/4 (r = 0 for lo, 1 for hi; j = lane % 16)
// of d block db, 4 columns per lane.  The swizzle of a row does not depend on t.
template <int D>
struct KtOffsets {
  int lo[D / 32];
  int hi[D / 32];
};
template <int D>
__device__ __forceinline__ KtOffsets<D> kt_offsets(int lane) {
  KtOffsets<D> o;
  const int half = lane >> 5;
  const int dsub = (lane >> 4) & 1;
  const int j = lane & 15;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int stored = swap23(8 * half + 4 * r + (j >> 2));  // LDS row of that tile row
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 4 * db + 2 * dsub + ((j & 3) >> 1);
      const int off = stored * D + (c ^ swz_k<D>(stored)) * 8 + (j & 1) * 4;
      if (r == 0) o.lo[db] = off; else o.hi[db] = off;
    }
  }
  return o;
}

// acc[db] += X^T F for a K-layout tile X (BN rows x D): lane (column l32 of the
// fragments' side, half h), d block db, register r holds d = 32db + 8(r/4) + 4h + r%4.
// The X^T operand (8 tile rows 16t + 8h + e for d = 32db + l32) comes from two
// transposing reads; fr[t] holds the matching 8 rows of the other operand.
template <int D, int BN>
__device__ __forceinline__ void kt_tile(const unsigned short* buf, const KtOffsets<D>& o, const bf16x8 (&fr)[BN / 16],
                                        f32x16 (&acc)[D / 32]) {
  int lo_off[D / 32], hi_off[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    lo_off[db] = fresh(o.lo[db]);
    hi_off[db] = fresh(o.hi[db]);
  }
#pragma unroll
  for (int t = 0; t < BN / 16; ++t) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint2 lo = lds_read_tr(buf + 16 * t * D + lo_off[db]);
      const uint2 hi = lds_read_tr(buf + 16 * t * D + hi_off[db]);
      acc[db] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), fr[t], acc[db]);
    }
  }
}

// Wait until this wave's LDS operations have completed and all but its N most
// recent vector-memory loads have landed.
template <int N>
__device__ __forceinline__ void wait_lgkm_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
}

// Barrier without a memory fence, for the mid-step switch of the two groups'
// roles: no LDS hazard crosses it (every buffer reuse is ordered by the
// end-of-step barrier), and a release fence here would wait for the tile fetch
// that has just been issued.
__device__ __forceinline__ void barrier_plain() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// End-of-step barrier of the tile ring: this wave's LDS reads have completed and
// all but its N most recent LDS-direct loads have landed before it arrives.  The
// empty asm keeps the compiler from moving memory accesses across; unlike a
// release fence it does not drain the loads still in flight.
template <int N>
__device__ __forceinline__ void barrier_ring() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0070 | N);  // lgkmcnt(0), vmcnt(N)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Barrier that orders LDS only: prefetches from global memory stay in flight.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace fa
