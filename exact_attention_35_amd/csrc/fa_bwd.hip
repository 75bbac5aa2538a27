// Backward kernels of exact attention for gfx950 (MI355X).
//
// The everydayai.blog flash-attention article ("Enter Flash Attention",
// point 2) states the strategy: the backward pass recomputes the attention
// tiles instead of storing the N x N matrix.  With P recomputed from the saved
// row log-sum-exp, the gradients of L = sum(dO * O) are
//
//   D_i = sum_k dO_ik O_ik      (= sum_j P_ij dP_ij)
//   dV  = P^T dO    dP = dO V^T    dS = P * (dP - D)
//   dQ  = scale dS K              dK = scale dS^T Q
//
// bf16 path, two kernels, in this order:
//   * bwd_dq_kernel: one workgroup owns 256 queries; each lane already holds
//     its query's dO row, so it first forms D and lse log2(e) (+inf for a row
//     with no visible key, so that its P is 0) and stores them as one float2
//     per row; it then streams K and V tiles through LDS and accumulates dQ in
//     registers (at d = 64, and for causal sequences of up to 2048 keys at
//     d = 128: bwd_dq_short_kernel, 128 queries and 4 waves per workgroup, two
//     or three workgroups per CU, the same arithmetic);
//   * bwd_dkdv_kernel: one workgroup owns 128 keys; it streams 64-query tiles
//     of Q and dO (and the stored row pairs) through LDS and accumulates dK,
//     dV in registers.
// The fp32 path forms the row pairs in a kernel of their own (bwd_prep_kernel).
// Each gradient is owned by exactly one workgroup, so there are no atomics
// and the results are deterministic; the price is that S and dP are
// recomputed by both the dK/dV and the dQ kernel (seven tile contractions per
// (query, key) tile pair instead of five).  Grouped-query heads: the dK/dV
// kernel writes each query head's fp32 dK, dV to the workspace and
// bwd_group_sum_kernel adds each group's heads in head order.
#include <math.h>

#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// fp32 path: stats[row] = (lse * log2 e, -D) with D = rowsum(dO * O).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ o, const float* __restrict__ dO,
                                                       const float* __restrict__ lse, float2* __restrict__ stats,
                                                       long long rows) {
  constexpr int TPR = D / 4;     // threads per row, 4 floats each
  constexpr int RPB = 256 / TPR;  // rows per block
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int part = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const float4 ov = *reinterpret_cast<const float4*>(o + row * D + part * 4);
    const float4 gv = *reinterpret_cast<const float4*>(dO + row * D + part * 4);
    acc = fmaf(ov.w, gv.w, fmaf(ov.z, gv.z, fmaf(ov.y, gv.y, ov.x * gv.x)));
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    const float l = lse[row];
    stats[row] = make_float2(l == -INFINITY ? INFINITY : l * kLog2e, -acc);
  }
}

__device__ __forceinline__ void buf_store16f(BufRes r, unsigned int byte_off, float a0, float a1, float a2, float a3) {
  u32x4 v;
  v[0] = __float_as_uint(a0);
  v[1] = __float_as_uint(a1);
  v[2] = __float_as_uint(a2);
  v[3] = __float_as_uint(a3);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 0);
}

// Store a [rows x D] gradient block held as MFMA accumulators with lane = row
// (row index `row`, half h) and register r of d block db at d = 32db + 8(r/4) + 4h + r%4,
// times `mul`, as fp32 or bf16.  Rows past the head are dropped by the range check.
template <int D>
__device__ __forceinline__ void store_grad_rows(void* base, size_t hoff, int N, int row, int half, int grad_bf16,
                                                const f32x16 (&acc)[D / 32], float mul) {
  if (grad_bf16) {
    const BufRes res = make_buf(static_cast<unsigned short*>(base) + hoff, (unsigned int)N * D * 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * half;
        uint2 pk;
        pk.x = (unsigned int)float_to_bf16_bits(acc[db][4 * i + 0] * mul) |
               ((unsigned int)float_to_bf16_bits(acc[db][4 * i + 1] * mul) << 16);
        pk.y = (unsigned int)float_to_bf16_bits(acc[db][4 * i + 2] * mul) |
               ((unsigned int)float_to_bf16_bits(acc[db][4 * i + 3] * mul) << 16);
        buf_store8(res, (unsigned int)(row * D + d0) * 2, pk);
      }
    }
  } else {
    const BufRes res = make_buf(static_cast<float*>(base) + hoff, (unsigned int)N * D * 4);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * db + 8 * i + 4 * half;
        buf_store16f(res, (unsigned int)(row * D + d0) * 4, acc[db][4 * i + 0] * mul, acc[db][4 * i + 1] * mul,
                     acc[db][4 * i + 2] * mul, acc[db][4 * i + 3] * mul);
      }
    }
  }
}

struct BwdBf16Args {
  const unsigned short* q;
  const unsigned short* k;
  const unsigned short* v;
  const unsigned short* dO;
  const unsigned short* o;    // the forward's output, for D (dQ kernel)
  const unsigned short* olo;  // its low-order part, or null
  const float* lse;           // the forward's row log-sum-exp (dQ kernel)
  float2* stats;  // per row: (lse log2 e, -D), written by the dQ kernel for the dK/dV kernel
  const unsigned char* mask;  // block-sparse 128x128 tile mask [nb, nb], or null
  int nb;
  void* dq;
  void* dk;
  void* dv;
  int grad_bf16;
  int BH;
  int group;    // query heads per K/V head (1: plain multi-head)
  int N;
  float c;      // |scale| * log2(e), clamped away from 0
  float scale;  // factor of dQ and dK
  int neg;      // scale < 0: the sign of Q (dQ kernel) or K (dK/dV kernel) is flipped on load
};

// ---------------------------------------------------------------------------
// dQ kernel: one workgroup = 256 queries of one (b, h), 8 waves of 32 queries,
// organised like the forward: waves w and w+4 share a SIMD and form groups A
// (waves 0-3) and B (4-7) that alternate an MFMA phase and a vector phase.
//   G(t): dQ^T += K(t-1)^T dS^T(t-1);  S^T(t) = K(t) Q^T;  dP^T(t) = V(t) dO^T
//   E(t): P = exp2(S c - lse log2 e) (0 where masked);  dS = P (dP - D)
// One query per lane: its lse and D are one register each.  K and V tiles
// (both in the K layout) arrive by LDS-direct loads into rings of three
// buffers: K one step ahead (group B), V two steps ahead (group A).
// ---------------------------------------------------------------------------
template <int D, int BN>
__device__ __forceinline__ void sched_dq_gemm() {
  constexpr int NKT = (BN / 16) * (D / 32);      // dQ MFMAs, two transposing reads each
  constexpr int NQK = 2 * (BN / 32) * (D / 16);  // S^T and dP^T MFMAs, one read each
#pragma unroll
  for (int i = 0; i < 3; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int i = 0; i < NKT - 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < NQK - 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// This lane's query: Q and dO rows as MFMA B fragments (Q negated when the scale
// is), D = rowsum(dO * O) with O taken as o + o_lo when the low-order part is given
// (each half-wave sums its half of the row), and lse log2 e; the pair (lse log2 e, -D)
// is also stored for the dK/dV kernel, which runs next.  Returns (lse log2 e, D);
// rows past N read zeros and get lse log2 e = +inf, so their P is 0, as is that of a
// row with no visible key.
template <int D>
__device__ __forceinline__ float2 dq_row_setup(const BwdBf16Args& a, BufRes qres, BufRes dores, size_t hoff,
                                               unsigned int head_bytes, int bh, int qrow, int half,
                                               bf16x8 (&qf)[D / 16], bf16x8 (&dof)[D / 16]) {
  const int N = a.N;
  {
    const unsigned int sign = a.neg ? 0x80008000u : 0u;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const unsigned int off = (unsigned int)(qrow * D + 16 * c + 8 * half) * 2;  // rows past N: zeros
      uint4 u = buf_load16(qres, off);
      u.x ^= sign;
      u.y ^= sign;
      u.z ^= sign;
      u.w ^= sign;
      qf[c] = as_bf16x8(u);
      dof[c] = as_bf16x8(buf_load16(dores, off));
    }
  }
  float dpart = 0.f;
  {
    const BufRes ores = make_buf(a.o + hoff, head_bytes);
    const bool with_lo = a.olo != nullptr;
    const BufRes lres = make_buf(with_lo ? a.olo + hoff : a.o + hoff, head_bytes);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const unsigned int off = (unsigned int)(qrow * D + 16 * c + 8 * half) * 2;  // rows past N: zeros
      const uint4 ov = buf_load16(ores, off);
      const uint4 lv = with_lo ? buf_load16(lres, off) : zero_uint4();
      const uint4 gv = as_uint4(dof[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = bf16_bits_to_float(bf16_lane_of(gv, e));
        dpart = fmaf(bf16_bits_to_float(bf16_lane_of(ov, e)), g,
                     fmaf(bf16_bits_to_float(bf16_lane_of(lv, e)), g, dpart));
      }
    }
  }
  const float dlt = xhalf_sum(dpart);
  float lse2 = INFINITY;
  if (qrow < N) {
    const float l = a.lse[(size_t)bh * N + qrow];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;  // +inf: a row with no visible key has P = 0
    if (half == 0) a.stats[(size_t)bh * N + qrow] = make_float2(lse2, -dlt);
  }
  return make_float2(lse2, dlt);
}

// Vector phase of the dQ kernels for key tile kt: P = exp2(S c - lse log2 e) and
// dS = P (dP - D), overwriting s, packed to bf16 MFMA fragments.  MASKED zeroes dS
// for keys past N and, causal, after the query (a separate copy, so that the common
// path has no per-element selects).
template <int BN, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void dq_make_ds(f32x16 (&s)[BN / 32], const f32x16 (&dp)[BN / 32], bf16x8 (&dsf)[BN / 16],
                                           int kt, int N, int qrow, int half, float c, float lse2, float dlt) {
#pragma unroll
  for (int b = 0; b < BN / 32; ++b) {
    // key = base + off with off = 16(r/8) + (r%8) a constant: compare off with per-lane bounds
    const int base = kt * BN + 32 * b + 8 * half;
    const int lim_n = N - base, lim_c = qrow - base;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[b][r], c, -lse2));
      float ds = p * (dp[b][r] - dlt);
      if (MASKED) {
        const int off = 16 * (r >> 3) + (r & 7);
        ds = (off >= lim_n || (CAUSAL && off > lim_c)) ? 0.f : ds;
      }
      s[b][r] = ds;
    }
  }
#pragma unroll
  for (int t2 = 0; t2 < BN / 16; ++t2) dsf[t2] = pack_bf16(s[t2 >> 1], 8 * (t2 & 1));
}

// (Block-sparse dQ runs on bwd_dq_short_kernel, whose 128 queries are one mask row.)
template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdBf16Args a) {
  using C = TileCfg<D, BN>;
  constexpr int BM = 256;
  constexpr int NSB = C::NSB;
  constexpr int NPT = C::NPT;
  constexpr int NDB = D / 32;
  constexpr int NW = 4;                         // waves of a group that load one tile
  constexpr int LPW = C::TILE * 2 / 1024 / NW;  // 1 KB loads per wave per tile
  __shared__ __align__(16) unsigned short kbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short kbuf_1[C::TILE];
  __shared__ __align__(16) unsigned short kbuf_2[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_1[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_2[C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int grp = w >> 2;
  const int wg = w & 3;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;
  const int nqt = (N + BM - 1) / BM;
  constexpr bool HR = !CAUSAL;  // head runs per XCD (grid_pos)
  const GridPos gp = CAUSAL ? grid_pos_causal(nqt, a.BH, 32) : grid_pos<HR>(nqt, a.BH);
  const int qt = CAUSAL ? nqt - 1 - gp.r : gp.r;  // longest rows first
  const int bh = gp.bh;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const size_t kvoff = (size_t)(bh / a.group) * (size_t)N * D;  // grouped-query: shared K/V head
  const unsigned int head_bytes = (unsigned int)N * D * 2;
  const BufRes qres = make_buf(a.q + hoff, head_bytes);
  const BufRes kres = make_buf(a.k + kvoff, head_bytes);
  const BufRes vres = make_buf(a.v + kvoff, head_bytes);
  const BufRes dores = make_buf(a.dO + hoff, head_bytes);

  const int q_first = qt * BM;
  // query blocks interleave between the groups so that causal work is balanced
  const int wave_q0 = q_first + 32 * (2 * wg + grp);
  const int qrow = wave_q0 + l32;
  const int wi = wg;  // this wave's share of a tile load
  unsigned short* const kb0 = kbuf_0;
  unsigned short* const kb1 = kbuf_1;
  unsigned short* const kb2 = kbuf_2;
  unsigned short* const vb0 = vbuf_0;
  unsigned short* const vb1 = vbuf_1;
  unsigned short* const vb2 = vbuf_2;
  const int kend = CAUSAL ? min(N, q_first + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  const int nsteps = ntiles;
  auto tile_at = [&](int t) __attribute__((always_inline)) -> int { return min(t, ntiles - 1); };
  auto need_mask = [&](int kt) __attribute__((always_inline)) -> bool {
    const int k_first = kt * BN;
    return (k_first + BN > N) || (CAUSAL && k_first + BN - 1 > wave_q0);
  };

  // Every tile buffer starts as zeros: K(-1) is read (times dS = 0) by the first
  // MFMA phase, and rows past N (which the range-checked loads may leave
  // unwritten) are multiplied by zeros, so they must hold finite values.
  for (int i = tid; i < C::TILE / 8; i += 512) {
    reinterpret_cast<uint4*>(kbuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(kbuf_1)[i] = zero_uint4();
    reinterpret_cast<uint4*>(kbuf_2)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_1)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_2)[i] = zero_uint4();
  }
  barrier_lds();
  if (ntiles > 0) {
    if (grp == 1) {
      dma_k<D, BN, NW>(kres, kb0, tile_at(0), wi, lane);
      wait_dma();
    } else {
      dma_k<D, BN, NW>(vres, vb0, tile_at(0), wi, lane);
      dma_k<D, BN, NW>(vres, vb1, tile_at(1), wi, lane);
    }
  }
  barrier_ring<LPW>();  // V(1) may still be landing

  bf16x8 qf[D / 16], dof[D / 16];
  const float2 row = dq_row_setup<D>(a, qres, dores, hoff, head_bytes, bh, qrow, half, qf, dof);
  const float lse2 = row.x, dlt = row.y;
  const KOffsets<D> ko = k_offsets<D>(l32, half);
  const KtOffsets<D> kto = kt_offsets<D>(lane);
  const float c = a.c;

  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = zero16();
  f32x16 s[NSB], dp[NSB];
  bf16x8 dsf[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) dsf[i] = as_bf16x8(zero_uint4());

  auto gemm_phase = [&](const unsigned short* kprev, const unsigned short* kcur, const unsigned short* vcur)
                        __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    kt_tile<D, BN>(kprev, kto, dsf, dqacc);
    qk_pair_tile<D, BN>(kcur, vcur, ko, qf, dof, s, dp);
    sched_dq_gemm<D, BN>();
    __builtin_amdgcn_s_setprio(0);
  };
  auto vector_phase = [&](int t) __attribute__((always_inline)) {
    const int kt = tile_at(t);
    if (need_mask(kt)) dq_make_ds<BN, CAUSAL, true>(s, dp, dsf, kt, N, qrow, half, c, lse2, dlt);
    else dq_make_ds<BN, CAUSAL, false>(s, dp, dsf, kt, N, qrow, half, c, lse2, dlt);
  };

  // Step t: buffers rotate with t mod 3.  kprev holds K(t-1), kcur K(t), vcur V(t);
  // group B fetches K(t+1) into knext, group A V(t+2) into vnext2.
  auto step = [&](int t, const unsigned short* kprev, const unsigned short* kcur, unsigned short* knext,
                  const unsigned short* vcur, unsigned short* vnext2) __attribute__((always_inline)) {
    const bool active = ntiles > 0 && t <= ntiles;
    if (grp == 0) {
      if (active) {
        dma_k<D, BN, NW>(vres, vnext2, tile_at(t + 2), wi, lane);
        gemm_phase(kprev, kcur, vcur);
      }
    } else {
      if (active) dma_k<D, BN, NW>(kres, knext, tile_at(t + 1), wi, lane);
      if (t >= 1 && t - 1 < ntiles) vector_phase(t - 1);
    }
    // No mid-step barrier: the ring buffers need just the end-of-step barrier (every
    // buffer written in step t was last read in step t - 1), and the two groups run
    // faster with their phases left to drift.
    if (grp == 0) {
      if (t < ntiles) vector_phase(t);
      wait_lgkm_vm<LPW>();  // V(t+1) has landed
    } else {
      if (active) gemm_phase(kprev, kcur, vcur);
      wait_lgkm_vm<0>();  // K(t+1) has landed
    }
    barrier_ring<15>();
  };
  // every wave runs the same steps (the barriers need it)
  for (int t = 0; nsteps > 0 && t <= nsteps; t += 3) {
    step(t, kb2, kb0, kb1, vb0, vb2);
    if (t + 1 <= nsteps) step(t + 1, kb0, kb1, kb2, vb1, vb0);
    if (t + 2 <= nsteps) step(t + 2, kb1, kb2, kb0, vb2, vb1);
  }
  wait_dma();  // no LDS-direct load may outlive the workgroup

  store_grad_rows<D>(a.dq, hoff, N, qrow, half, a.grad_bf16, dqacc, a.scale);
}

// ---------------------------------------------------------------------------
// dQ kernel for short key ranges: one workgroup = 128 queries of one
// (b, h), 4 waves of 32 queries, one per SIMD.  Each wave runs G(t) and then E(t)
// of the same step itself (the arithmetic of bwd_dq_kernel, so the results are the
// same bit for bit for the same tile size).  K and V tiles go through rings of
// three buffers, K one step and V two steps ahead.  Several workgroups share a CU,
// so that one's prologue, pipeline fill and epilogue overlap another's steady
// state: two at d = 128 (48 KB of LDS), three at d = 64, where 32-key tiles (24 KB)
// let the kernel be held to 168 registers.
// ---------------------------------------------------------------------------
template <int D, int BN, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 1, 8)))
void bwd_dq_short_kernel(BwdBf16Args a) {
  using C = TileCfg<D, BN>;
  constexpr int BM = 128;
  constexpr int NSB = C::NSB;
  constexpr int NPT = C::NPT;
  constexpr int NDB = D / 32;
  constexpr int LPW = C::TILE * 2 / 1024 / 4;  // 1 KB loads per wave per tile
  __shared__ __align__(16) unsigned short kbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short kbuf_1[C::TILE];
  __shared__ __align__(16) unsigned short kbuf_2[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_1[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_2[C::TILE];
  extern __shared__ __align__(16) unsigned short col_list[];  // SPARSE: kept columns of the mask row
  __shared__ int list_len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;
  const int nqt = (N + BM - 1) / BM;  // = the mask's row count: one workgroup per mask row
  constexpr bool HR = SPARSE || !CAUSAL;  // head runs per XCD (grid_pos)
  const GridPos gp = (CAUSAL && !SPARSE) ? grid_pos_causal(nqt, a.BH, 32 * (D == 64 ? 3 : 2))
                                         : grid_pos<HR>(nqt, a.BH);
  const int qt = CAUSAL ? nqt - 1 - gp.r : gp.r;  // longest rows first
  const int bh = gp.bh;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const size_t kvoff = (size_t)(bh / a.group) * (size_t)N * D;  // grouped-query: shared K/V head
  const unsigned int head_bytes = (unsigned int)N * D * 2;
  const BufRes qres = make_buf(a.q + hoff, head_bytes);
  const BufRes kres = make_buf(a.k + kvoff, head_bytes);
  const BufRes vres = make_buf(a.v + kvoff, head_bytes);
  const BufRes dores = make_buf(a.dO + hoff, head_bytes);

  const int q_first = qt * BM;
  const int wave_q0 = q_first + 32 * w;
  const int qrow = wave_q0 + l32;
  const int wi = __builtin_amdgcn_readfirstlane(w);  // this wave's share of a tile load
  int ntiles;
  if (SPARSE) {
    // block-sparse: wave 0 lists the key columns its mask row keeps (128 keys each)
    constexpr int R = 128 / BN;  // key tiles per mask column
    const int nb = a.nb;
    if (w == 0) {
      const int cnt = list_kept(a.mask + (size_t)qt * nb, 1, 0, CAUSAL ? qt + 1 : nb, col_list, lane);
      if (lane == 0) list_len = cnt;
    }
    __syncthreads();
    // R tiles per listed column, minus those of the last column past N
    const int len = list_len;
    ntiles = len * R;
    if (len > 0 && col_list[len - 1] == nb - 1) ntiles -= R - ((N - (nb - 1) * 128 + BN - 1) / BN);
  } else {
    const int kend = CAUSAL ? min(N, q_first + BM) : N;
    ntiles = (kend + BN - 1) / BN;
  }
  auto tile_at = [&](int t) __attribute__((always_inline)) -> int {  // steps past the end repeat the last tile
    const int tt = min(t, ntiles - 1);
    if (!SPARSE) return tt;
    constexpr int R = 128 / BN;
    return (int)col_list[tt / R] * R + tt % R;
  };
  auto need_mask = [&](int kt) __attribute__((always_inline)) -> bool {
    const int k_first = kt * BN;
    return (k_first + BN > N) || (CAUSAL && k_first + BN - 1 > wave_q0);
  };

  // Every tile buffer starts as zeros: K(-1) is read (times dS = 0) by the first
  // step, and rows past N (which the range-checked loads may leave unwritten) are
  // multiplied by zeros, so they must hold finite values.
  for (int i = tid; i < C::TILE / 8; i += 256) {
    reinterpret_cast<uint4*>(kbuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(kbuf_1)[i] = zero_uint4();
    reinterpret_cast<uint4*>(kbuf_2)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_1)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_2)[i] = zero_uint4();
  }
  barrier_lds();
  if (ntiles > 0) {
    dma_k<D, BN, 4>(kres, kbuf_0, tile_at(0), wi, lane);
    dma_k<D, BN, 4>(vres, vbuf_0, tile_at(0), wi, lane);
    dma_k<D, BN, 4>(vres, vbuf_1, tile_at(1), wi, lane);
  }
  barrier_ring<LPW>();  // K(0) and V(0) have landed; V(1) may still be landing

  bf16x8 qf[D / 16], dof[D / 16];
  const float2 row = dq_row_setup<D>(a, qres, dores, hoff, head_bytes, bh, qrow, half, qf, dof);
  const float lse2 = row.x, dlt = row.y;
  const KOffsets<D> ko = k_offsets<D>(l32, half);
  const KtOffsets<D> kto = kt_offsets<D>(lane);
  const float c = a.c;

  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = zero16();
  f32x16 s[NSB], dp[NSB];
  bf16x8 dsf[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) dsf[i] = as_bf16x8(zero_uint4());

  // Step t: buffers rotate with t mod 3; kprev holds K(t-1), kcur K(t), vcur V(t).
  // The wave fetches K(t+1) into knext and V(t+2) into vnext2, runs G(t) and E(t),
  // and ends the step once K(t+1) has landed everywhere (V(t+2) may still be
  // landing).  At t = 0 the dQ product uses dS = 0; at t = ntiles the S and dP of a
  // repeated tile are never used.
  auto step = [&](int t, const unsigned short* kprev, const unsigned short* kcur, unsigned short* knext,
                  const unsigned short* vcur, unsigned short* vnext2) __attribute__((always_inline)) {
    dma_k<D, BN, 4>(kres, knext, tile_at(t + 1), wi, lane);
    dma_k<D, BN, 4>(vres, vnext2, tile_at(t + 2), wi, lane);
    kt_tile<D, BN>(kprev, kto, dsf, dqacc);
    qk_pair_tile<D, BN>(kcur, vcur, ko, qf, dof, s, dp);
    sched_dq_gemm<D, BN>();
    if (t < ntiles) {
      const int kt = tile_at(t);
      if (need_mask(kt)) dq_make_ds<BN, CAUSAL, true>(s, dp, dsf, kt, N, qrow, half, c, lse2, dlt);
      else dq_make_ds<BN, CAUSAL, false>(s, dp, dsf, kt, N, qrow, half, c, lse2, dlt);
    }
    barrier_ring<LPW>();
  };
  // a block-sparse row without any kept tile has dQ = 0 (its row statistics are stored)
  for (int t = 0; ntiles > 0 && t <= ntiles; t += 3) {
    step(t, kbuf_2, kbuf_0, kbuf_1, vbuf_0, vbuf_2);
    if (t + 1 <= ntiles) step(t + 1, kbuf_0, kbuf_1, kbuf_2, vbuf_1, vbuf_0);
    if (t + 2 <= ntiles) step(t + 2, kbuf_1, kbuf_2, kbuf_0, vbuf_2, vbuf_1);
  }
  wait_dma();  // no LDS-direct load may outlive the workgroup

  store_grad_rows<D>(a.dq, hoff, N, qrow, half, a.grad_bf16, dqacc, a.scale);
}

// ---------------------------------------------------------------------------
// dK/dV kernel: one workgroup = 128 keys of one (b, h).  Waves w and w+4 share
// a SIMD and the 32 keys 32w .. 32w+31; they split the work by role:
//   score wave (w < 4): S = Q K^T and dP = dO V^T for its keys (K, V as MFMA B
//     fragments in VGPRs, one key per lane), then P = exp2(S c - lse log2 e)
//     and dS = P (dP - D), packed to bf16 and handed over through LDS;
//   gradient wave (w >= 4): dV^T += dO^T P and dK^T += Q^T dS for the same keys,
//     the dO^T / Q^T operands read from the tiles with transposing LDS reads.
// Step i, phase a: the score waves hand over dS(i) and run the S MFMAs of tile
// i+1 while the gradient waves run dV += dO(i)^T P(i); phase b: the score waves
// compute P(i+1) interleaved with the dP MFMAs of tile i+1 and hand over P(i+1)
// while the gradient waves fetch tile i+2 and run dK += Q(i)^T dS(i).  Q and dO tiles (64 queries, K layout)
// and their (lse log2 e, -D) rows sit in rings of three buffers.
// ---------------------------------------------------------------------------
// MFMA / LDS-read interleave of an MFMA phase (masks: 0x8 MFMA, 0x100 LDS read):
// PRE reads issue first, then after each MFMA the reads of a later one, so
// that LDS latency hides behind the MFMAs.  N1 MFMAs take one read each.
template <int N1>
__device__ __forceinline__ void sched_one_read_per_mfma() {
#pragma unroll
  for (int i = 0; i < 6; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int i = 0; i < N1 - 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < 6; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// PRE single reads first (operands held for the whole phase), then N2 MFMAs
// that take two reads each, three MFMAs ahead.
template <int PRE, int N2>
__device__ __forceinline__ void sched_two_reads_per_mfma() {
#pragma unroll
  for (int i = 0; i < PRE + 6; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int i = 0; i < N2 - 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

template <int D, int KG>
struct DkvCfg : TileCfg<D, 64> {
  static constexpr int BK = 32 * KG;                   // keys per workgroup
  static constexpr int BQ = 64;                        // queries per tile
  static constexpr int LPW = BQ * D * 2 / 1024 / KG;  // 1 KB loads per gradient wave and Q (or dO) tile
};

// KG key groups of 32 keys, each served by a score wave and a gradient wave: KG = 4
// (128 keys, 512 threads) puts the two waves of a group on one SIMD; KG = 2 (64 keys,
// 256 threads, at d = 64 two workgroups per CU) puts every wave on a SIMD of its own.
// Block-sparse (SPARSE): the workgroup's keys lie in one mask column; it visits the
// 64-query tiles of the mask rows that keep that column.
template <int D, bool CAUSAL, bool SPARSE, int KG>
__global__ __launch_bounds__(128 * KG) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(BwdBf16Args a) {
  using C = DkvCfg<D, KG>;
  constexpr int BQ = C::BQ;
  constexpr int NSB = C::NSB;  // 32-query blocks per tile
  constexpr int NPT = C::NPT;  // 16-query fragments per tile
  constexpr int NDB = D / 32;
  __shared__ __align__(16) unsigned short qbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short qbuf_1[C::TILE];
  __shared__ __align__(16) unsigned short qbuf_2[C::TILE];
  __shared__ __align__(16) unsigned short obuf_0[C::TILE];
  __shared__ __align__(16) unsigned short obuf_1[C::TILE];
  __shared__ __align__(16) unsigned short obuf_2[C::TILE];
  __shared__ __align__(16) float2 st_0[BQ];
  __shared__ __align__(16) float2 st_1[BQ];
  __shared__ __align__(16) float2 st_2[BQ];
  __shared__ __align__(16) uint4 xch[KG][2 * NPT][64];  // per key group: P then dS fragments, per lane
  extern __shared__ __align__(16) unsigned short row_list[];  // SPARSE: mask rows that keep this column
  __shared__ int row_len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: role branches are scalar
  const int sw = w % KG;      // key group (with KG = 4 also the SIMD)
  const bool score = w < KG;  // role
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;
  constexpr bool HR = SPARSE || !CAUSAL;  // head runs per XCD (grid_pos)
  const GridPos gp = (CAUSAL && !SPARSE) ? grid_pos_causal((N + C::BK - 1) / C::BK, a.BH, 32 * (4 / KG))
                                         : grid_pos<HR>((N + C::BK - 1) / C::BK, a.BH);
  const int kt = gp.r;  // causal: small kt = most query tiles, launched first
  const int bh = gp.bh;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const unsigned int head_bytes = (unsigned int)N * D * 2;
  const BufRes qres = make_buf(a.q + hoff, head_bytes);
  const BufRes dores = make_buf(a.dO + hoff, head_bytes);
  const BufRes sres = make_buf(a.stats + (size_t)bh * N, (unsigned int)N * 8);
  const int k0 = kt * C::BK;
  const int wave_k0 = k0 + 32 * sw;
  const int mykey = wave_k0 + l32;
  const int nqt = (N + BQ - 1) / BQ;
  const int t_first = CAUSAL ? k0 / BQ : 0;
  int T;  // query tiles this workgroup visits
  if (SPARSE) {
    const int nb = a.nb;
    const int mcol = k0 >> 7;  // the mask column of this workgroup's keys
    if (w == 0) {
      const int cnt = list_kept(a.mask + mcol, (size_t)nb, CAUSAL ? mcol : 0, nb, row_list, lane);
      if (lane == 0) row_len = cnt;
    }
    __syncthreads();
    const int len = row_len;
    T = 2 * len;  // two 64-query tiles per mask row, but none past N
    if (len > 0 && row_list[len - 1] == nb - 1 && N <= (nb - 1) * 128 + BQ) T -= 1;
  } else {
    T = nqt - t_first;  // >= 1: k0 < N
  }
  // query tile of step i (steps past the list stay in range; their tiles are masked)
  auto tile_q = [&](int i) __attribute__((always_inline)) -> int {
    if (!SPARSE) return t_first + i;
    const int j = min(i >> 1, max(row_len - 1, 0));
    return (int)row_list[j] * 2 + (i & 1);
  };

  // tile i into buffer set i % 3, by the gradient waves
  auto fetch = [&](int i, unsigned short* qb, unsigned short* ob, float2* st) __attribute__((always_inline)) {
    const int tq = tile_q(i);
    dma_k<D, BQ, KG>(qres, qb, tq, sw, lane);
    dma_k<D, BQ, KG>(dores, ob, tq, sw, lane);
    if (sw == 0) {
      // the 64 rows' (lse log2 e, -D) pairs regrouped per four rows: LDS dword 8g + e holds
      // lse log2 e of row 4g + e for e < 4 and -D of row 4g + e - 4 for e >= 4, so that
      // one 16-byte read gives four rows' -D, the initial dP accumulator (rows past N: zeros)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int j = 64 * m + lane;
        const int row = 4 * (j >> 3) + (j & 3);
        const unsigned int off = (unsigned int)((tq * BQ + row) * 8 + 4 * ((j >> 2) & 1));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, (lds_void_t*)(reinterpret_cast<float*>(st) + 64 * m), 4, off,
                                                 0, 0, 0);
      }
    }
  };
  constexpr int LOADS = 2 * C::LPW + 2;  // loads of one fetch by gradient wave 0 (the others: two fewer)
  static_assert(LOADS < 16, "vmcnt field of the waits below");

  // Every buffer starts as zeros: rows past N (which the range-checked loads may
  // leave unwritten) are multiplied by P = dS = 0 and must hold finite values.
  for (int i = tid; i < C::TILE / 8; i += 128 * KG) {
    reinterpret_cast<uint4*>(qbuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(qbuf_1)[i] = zero_uint4();
    reinterpret_cast<uint4*>(qbuf_2)[i] = zero_uint4();
    reinterpret_cast<uint4*>(obuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(obuf_1)[i] = zero_uint4();
    reinterpret_cast<uint4*>(obuf_2)[i] = zero_uint4();
  }
  if (tid < BQ) st_0[tid] = st_1[tid] = st_2[tid] = make_float2(0.f, 0.f);
  barrier_lds();
  if (!score && T > 0) {
    fetch(0, qbuf_0, obuf_0, st_0);
    if (T > 1) {
      fetch(1, qbuf_1, obuf_1, st_1);
      if (sw == 0) wait_dma_but<LOADS>(); else wait_dma_but<LOADS - 2>();  // tile 1 may still be landing
    } else {
      wait_dma();
    }
  }
  barrier_ring<15>();

  const float c = a.c;
  if (score) {
    // ---- score wave: K and V rows of this lane's key as MFMA B fragments
    bf16x8 kf[D / 16], vf[D / 16];
    {
      const size_t kvoff = (size_t)(bh / a.group) * (size_t)N * D;  // grouped-query: shared K/V head
      const BufRes kres = make_buf(a.k + kvoff, head_bytes);
      const BufRes vres = make_buf(a.v + kvoff, head_bytes);
      const unsigned int sign = a.neg ? 0x80008000u : 0u;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const unsigned int off = (unsigned int)(mykey * D + 16 * cc + 8 * half) * 2;  // keys past N: zeros
        uint4 u = buf_load16(kres, off);
        u.x ^= sign;
        u.y ^= sign;
        u.z ^= sign;
        u.w ^= sign;
        kf[cc] = as_bf16x8(u);
        vf[cc] = as_bf16x8(buf_load16(vres, off));
      }
    }
    const KOffsets<D> ko = k_offsets<D>(l32, half);
    f32x16 s[NSB], dp[NSB];
    bf16x8 pf[NPT], dsf[NPT];
    // S = K Q^T of one tile (from zero)
    auto s_mfma = [&](const unsigned short* qb) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int b = 0; b < NSB; ++b) s[b] = zero16();
      qk_ring_tile<D, BQ>(qb, ko, kf, s);
      sched_one_read_per_mfma<NSB * (D / 16)>();
      __builtin_amdgcn_s_setprio(0);
    };
    // P of tile i and dP(i) - D = V dO^T - D together, in one fixed instruction order: dp
    // starts at -D (read from LDS straight into the accumulator), then each dP MFMA is
    // followed by the LDS operand read of the MFMA AHEAD places later and by the
    // exponentials of PER scores, with scheduling fences between the slices, so that
    // the wave's vector work issues while its own MFMAs run.  P (register r of block b
    // is query 32b + acc_row_swapped(r, half)) goes to s (fp32, for dS) and to pf (bf16,
    // for the handover).  The masked variant is a separate copy so that the common path
    // has no per-element selects.
    auto p_dp_fused = [&](int q0, const float2* st, const unsigned short* ob, auto mask_tag)
                          __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(mask_tag)::value;
      constexpr int NM = NSB * (D / 16);  // dP MFMAs: chunk m / NSB, block m % NSB
      constexpr int NE = 16 * NSB;        // P elements per lane
      constexpr int PER = NE / NM;
      constexpr int AHEAD = 4;
      static_assert(PER * NM == NE, "whole slices of P per MFMA");
      f32x4 lq[NSB][4];
#pragma unroll
      for (int b = 0; b < NSB; ++b) {
        const f32x4* src = reinterpret_cast<const f32x4*>(st + 32 * b + 8 * half);
        dp[b] = __builtin_shufflevector(__builtin_shufflevector(src[1], src[3], 0, 1, 2, 3, 4, 5, 6, 7),
                                        __builtin_shufflevector(src[9], src[11], 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2,
                                        3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        lq[b][0] = src[0];
        lq[b][1] = src[2];
        lq[b][2] = src[8];
        lq[b][3] = src[10];
      }
      int o[D / 16];
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) o[cc] = fresh(ko.off[cc]);
      bf16x8 ring[AHEAD];
#pragma unroll
      for (int m = 0; m < AHEAD; ++m) ring[m] = lds_bf16x8(ob + 32 * (m % NSB) * D + o[m / NSB]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const bf16x8 x = ring[m % AHEAD];
        if (m + AHEAD < NM) ring[m % AHEAD] = lds_bf16x8(ob + 32 * ((m + AHEAD) % NSB) * D + o[(m + AHEAD) / NSB]);
        dp[m % NSB] = mfma32(x, vf[m / NSB], dp[m % NSB]);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int k = m * PER + e;
          const int b = k >> 4, r = k & 15;
          const float lv = lq[b][2 * (r >> 3) + ((r & 7) >> 2)][r & 3];
          float p = __builtin_amdgcn_exp2f(fmaf(s[b][r], c, -lv));
          if (MASKED) {
            // query = base + off with off = 16(r/8) + (r%8) a constant
            const int base = q0 + 32 * b + 8 * half;
            const int off = 16 * (r >> 3) + (r & 7);
            const bool hide = off >= N - base || (CAUSAL && off < mykey - base);
            p = hide ? 0.f : p;
          }
          s[b][r] = p;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int t2 = 0; t2 < NPT; ++t2) pf[t2] = pack_bf16(s[t2 >> 1], 8 * (t2 & 1));
    };
    auto p_dp = [&](int i, const float2* st, const unsigned short* ob) __attribute__((always_inline)) {
      const int q0 = i < T ? tile_q(i) * BQ : N;  // past the last tile: everything masked
      if ((q0 + BQ > N) || (CAUSAL && q0 < wave_k0 + 31)) p_dp_fused(q0, st, ob, std::true_type{});
      else p_dp_fused(q0, st, ob, std::false_type{});
    };
    // dS = P (dP - D); a masked P is 0, and so is its dS (dP - D is finite)
    auto ds_vector = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < NSB; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[b][r] *= s[b][r];
      }
#pragma unroll
      for (int t2 = 0; t2 < NPT; ++t2) dsf[t2] = pack_bf16(dp[t2 >> 1], 8 * (t2 & 1));
    };
    // Step i: phase a computes and hands over dS(i), then runs S(i+1); phase b
    // computes and hands over P(i+1), then runs dP(i+1).  The two phases carry the
    // same MFMA count, and each SIMD's gradient wave adds 16 MFMAs to both.
    // Unconditional, so that no value lives across a handover: at i + 1 = T the tile
    // is past N and every P (hence dS) of it is masked to zero.
    auto step = [&](int i, const unsigned short* qnxt, const unsigned short* onxt, const float2* snxt)
                    __attribute__((always_inline)) {
      ds_vector();
#pragma unroll
      for (int t2 = 0; t2 < NPT; ++t2) xch[sw][NPT + t2][lane] = as_uint4(dsf[t2]);
      s_mfma(qnxt);
      barrier_ring<15>();  // the dS handover writes have completed
      p_dp(i + 1, snxt, onxt);
#pragma unroll
      for (int t2 = 0; t2 < NPT; ++t2) xch[sw][t2][lane] = as_uint4(pf[t2]);
      barrier_ring<15>();  // the P handover writes have completed
    };
    s_mfma(qbuf_0);
    p_dp(0, st_0, obuf_0);
#pragma unroll
    for (int t2 = 0; t2 < NPT; ++t2) xch[sw][t2][lane] = as_uint4(pf[t2]);
    barrier_ring<15>();
    for (int i = 0; i < T; i += 3) {
      step(i, qbuf_1, obuf_1, st_1);
      if (i + 1 < T) step(i + 1, qbuf_2, obuf_2, st_2);
      if (i + 2 < T) step(i + 2, qbuf_0, obuf_0, st_0);
    }
  } else {
    // ---- gradient wave: dV^T and dK^T accumulators (lane = key, registers = d)
    const KtOffsets<D> kto = kt_offsets<D>(lane);
    f32x16 dvacc[NDB], dkacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      dvacc[i] = zero16();
      dkacc[i] = zero16();
    }
    // acc^T += X^T F for one tile, F the handed-over fragments at xch[sw][f0 ..]
    auto grad_mfma = [&](const unsigned short* xb, int f0, f32x16 (&acc)[NDB]) __attribute__((always_inline)) {
      bf16x8 xf[NPT];
#pragma unroll
      for (int t2 = 0; t2 < NPT; ++t2) xf[t2] = as_bf16x8(xch[sw][f0 + t2][lane]);
      __builtin_amdgcn_s_setprio(1);
      kt_tile<D, BQ>(xb, kto, xf, acc);
      sched_two_reads_per_mfma<NPT, NPT * NDB>();
      __builtin_amdgcn_s_setprio(0);
    };
    // Step i: phase a dV += dO(i)^T P(i); phase b fetch tile i+2, dK += Q(i)^T dS(i)
    auto step = [&](int i, const unsigned short* qcur, const unsigned short* ocur, unsigned short* qfar,
                    unsigned short* ofar, float2* sfar) __attribute__((always_inline)) {
      grad_mfma(ocur, 0, dvacc);
      barrier_ring<15>();
      if (i + 2 < T) fetch(i + 2, qfar, ofar, sfar);
      grad_mfma(qcur, NPT, dkacc);
      wait_lgkm_vm<0>();  // tile i+2 has landed
      barrier_ring<15>();
    };
    wait_dma();  // tile 1 has landed
    barrier_ring<15>();
    for (int i = 0; i < T; i += 3) {
      step(i, qbuf_0, obuf_0, qbuf_2, obuf_2, st_2);
      if (i + 1 < T) step(i + 1, qbuf_1, obuf_1, qbuf_0, obuf_0, st_0);
      if (i + 2 < T) step(i + 2, qbuf_2, obuf_2, qbuf_1, obuf_1, st_1);
    }
    wait_dma();
    store_grad_rows<D>(a.dv, hoff, N, mykey, half, a.grad_bf16, dvacc, 1.f);
    store_grad_rows<D>(a.dk, hoff, N, mykey, half, a.grad_bf16, dkacc, a.scale);
  }
}

// ---------------------------------------------------------------------------
// fp32 backward: plain correctness kernels (no MFMA), deterministic.
//   dK/dV: one thread per key, the query rows staged through LDS.
//   dQ:    one thread per query, the key rows staged through LDS.
// ---------------------------------------------------------------------------
struct BwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* dO;
  const float* lse;
  const float2* stats;  // (lse log2 e, -D) per row; D is used here
  float* dq;
  float* dk;
  float* dv;
  int BH;
  int group;  // query heads per K/V head
  int N;
  float scale;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void bwd_f32_dkdv_kernel(BwdF32Args a) {
  constexpr int BK = 64;  // keys per workgroup (one per thread)
  constexpr int BQ = 16;  // query rows staged per step
  __shared__ float kk[BK * (D + 1)];
  __shared__ float vv[BK * (D + 1)];
  __shared__ float qs[BQ * D];
  __shared__ float dos[BQ * D];
  __shared__ float ls[BQ], dl[BQ];
  const int tid = threadIdx.x;
  const int N = a.N;
  const int kt = (int)(blockIdx.x / a.BH);
  const int bh = (int)(blockIdx.x % a.BH);
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(bh / a.group) * N * D;
  const int k0 = kt * BK;
  for (int idx = tid; idx < BK * D; idx += 64) {
    const int row = idx / D, col = idx % D;
    const int key = k0 + row;
    kk[row * (D + 1) + col] = key < N ? a.k[kvoff + (size_t)key * D + col] : 0.f;
    vv[row * (D + 1) + col] = key < N ? a.v[kvoff + (size_t)key * D + col] : 0.f;
  }
  const int key = k0 + tid;
  float gk[D], gv[D];
#pragma unroll
  for (int i = 0; i < D; ++i) gk[i] = gv[i] = 0.f;
  const int qstart = CAUSAL ? (k0 / BQ) * BQ : 0;
  for (int q0 = qstart; q0 < N; q0 += BQ) {
    __syncthreads();
    for (int idx = tid; idx < BQ * D; idx += 64) {
      const int row = q0 + idx / D;
      qs[idx] = row < N ? a.q[hoff + (size_t)row * D + idx % D] : 0.f;
      dos[idx] = row < N ? a.dO[hoff + (size_t)row * D + idx % D] : 0.f;
    }
    if (tid < BQ) {
      const int row = q0 + tid;
      ls[tid] = row < N ? a.lse[hoff / D + row] : -INFINITY;
      dl[tid] = row < N ? -a.stats[hoff / D + row].y : 0.f;
    }
    __syncthreads();
    if (key < N) {
      for (int i = 0; i < BQ; ++i) {
        const int qi = q0 + i;
        if (qi >= N || (CAUSAL && key > qi) || ls[i] == -INFINITY) continue;
        float sd = 0.f, dpd = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) {
          sd = fmaf(qs[i * D + t], kk[tid * (D + 1) + t], sd);
          dpd = fmaf(dos[i * D + t], vv[tid * (D + 1) + t], dpd);
        }
        const float p = expf(sd * a.scale - ls[i]);
        const float ds = p * (dpd - dl[i]);
#pragma unroll
        for (int t = 0; t < D; ++t) {
          gv[t] = fmaf(p, dos[i * D + t], gv[t]);
          gk[t] = fmaf(ds, qs[i * D + t], gk[t]);
        }
      }
    }
  }
  if (key < N) {
#pragma unroll
    for (int t = 0; t < D; ++t) {
      a.dk[hoff + (size_t)key * D + t] = gk[t] * a.scale;
      a.dv[hoff + (size_t)key * D + t] = gv[t];
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void bwd_f32_dq_kernel(BwdF32Args a) {
  constexpr int BQ = 64;
  constexpr int BK = 16;
  __shared__ float kk[BK * D];
  __shared__ float vv[BK * D];
  __shared__ float dos[BQ * (D + 1)];  // each thread's dO row (stride D + 1: no bank conflicts)
  const int tid = threadIdx.x;
  const int N = a.N;
  const int qt = (int)(blockIdx.x / a.BH);
  const int bh = (int)(blockIdx.x % a.BH);
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(bh / a.group) * N * D;
  const int qi = qt * BQ + tid;
  const bool in = qi < N;
  float qv[D], g[D];
  float* const dov = dos + tid * (D + 1);
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qv[t] = in ? a.q[hoff + (size_t)qi * D + t] : 0.f;
    dov[t] = in ? a.dO[hoff + (size_t)qi * D + t] : 0.f;
    g[t] = 0.f;
  }
  const float l = in ? a.lse[hoff / D + qi] : -INFINITY;
  const float dl = in ? -a.stats[hoff / D + qi].y : 0.f;
  const int kend = CAUSAL ? min(N, qt * BQ + BQ) : N;
  for (int k0 = 0; k0 < kend; k0 += BK) {
    __syncthreads();
    for (int idx = tid; idx < BK * D; idx += 64) {
      const int row = k0 + idx / D;
      kk[idx] = row < N ? a.k[kvoff + (size_t)row * D + idx % D] : 0.f;
      vv[idx] = row < N ? a.v[kvoff + (size_t)row * D + idx % D] : 0.f;
    }
    __syncthreads();
    if (in && l != -INFINITY) {
      for (int j = 0; j < BK; ++j) {
        const int key = k0 + j;
        if (key >= N || (CAUSAL && key > qi)) break;
        float sd = 0.f, dpd = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) {
          sd = fmaf(qv[t], kk[j * D + t], sd);
          dpd = fmaf(dov[t], vv[j * D + t], dpd);
        }
        const float p = expf(sd * a.scale - l);
        const float ds = p * (dpd - dl);
        // read the key row from LDS again rather than keep it in D registers since the dot
        // product (at d = 128 that would spill)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < D; ++t) g[t] = fmaf(ds, kk[j * D + t], g[t]);
      }
    }
  }
  if (in) {
#pragma unroll
    for (int t = 0; t < D; ++t) a.dq[hoff + (size_t)qi * D + t] = g[t] * a.scale;
  }
}

// ---------------------------------------------------------------------------
// Grouped-query dK/dV: the per-query-head fp32 gradients [B, H, N, d] are summed
// over each run of `group` consecutive heads into [B, H_kv, N, d], in head order
// (deterministic), and written as fp32 or bf16.  HBM-bound: one thread per four
// output elements, float4 loads of the group's partials.
// ---------------------------------------------------------------------------
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float* __restrict__ pk, const float* __restrict__ pv,
                                                            void* __restrict__ dk, void* __restrict__ dv,
                                                            long long quads, long long head_quads, int group) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * quads) return;
  const bool is_v = i >= quads;
  const long long e = is_v ? i - quads : i;  // quad index in [B, H_kv, N, d / 4]
  const long long kvh = e / head_quads;
  const long long src = (kvh * group) * head_quads + (e - kvh * head_quads);
  const float4* p = reinterpret_cast<const float4*>(is_v ? pv : pk) + src;
  float4 acc = p[0];
  for (int j = 1; j < group; ++j) {
    const float4 t = p[(long long)j * head_quads];
    acc.x += t.x;
    acc.y += t.y;
    acc.z += t.z;
    acc.w += t.w;
  }
  void* out = is_v ? dv : dk;
  if (BF16_OUT) {
    uint2 pk2;
    pk2.x = (unsigned int)float_to_bf16_bits(acc.x) | ((unsigned int)float_to_bf16_bits(acc.y) << 16);
    pk2.y = (unsigned int)float_to_bf16_bits(acc.z) | ((unsigned int)float_to_bf16_bits(acc.w) << 16);
    reinterpret_cast<uint2*>(out)[e] = pk2;
  } else {
    reinterpret_cast<float4*>(out)[e] = acc;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static void launch_group_sum(const BwdParams& p, hipStream_t stream) {
  const long long head_quads = (long long)p.N * p.d / 4;
  const long long quads = (long long)p.B * p.Hkv * head_quads;
  const unsigned blocks = (unsigned)((2 * quads + 255) / 256);
  if (p.grad_dtype == 1)
    hipLaunchKernelGGL((bwd_group_sum_kernel<true>), dim3(blocks), dim3(256), 0, stream, p.part_k, p.part_v, p.dk,
                       p.dv, quads, head_quads, p.H / p.Hkv);
  else
    hipLaunchKernelGGL((bwd_group_sum_kernel<false>), dim3(blocks), dim3(256), 0, stream, p.part_k, p.part_v, p.dk,
                       p.dv, quads, head_quads, p.H / p.Hkv);
}

template <int D>
static void launch_prep_f32(const BwdParams& p, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 4);
  const long long rows = (long long)p.B * p.H * p.N;
  const unsigned blocks = (unsigned)((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(blocks), dim3(256), 0, stream, static_cast<const float*>(p.o),
                     static_cast<const float*>(p.dO), p.lse, reinterpret_cast<float2*>(p.stats), rows);
}

// When bwd_dq_short_kernel serves the dQ of a dense bf16 backward (measured on MI355X,
// bf16, 12-16 heads, whole backward against bwd_dq_kernel, interleaved on one box): at
// d = 64 (32-key tiles, three workgroups per CU) always, causal or not (9-10% faster at
// causal N = 512-2048, 4-7% without masking, 3-4% at 4K-8K, 14% on a grid of 256
// workgroups, 1-2% at 16K-64K); at d = 128 (two per CU) for causal N <= 2048 (0-3%
// faster, 12% on a grid of 128 workgroups), where without causal masking it lost 4%.
constexpr int kShortCausalN = 2048;

constexpr int kDkvPairN = 2048;  // d = 64: 64-key dK/dV workgroups up to this N (twice it without causal masking)

// dK/dV on workgroups of KG key groups (32 keys each)
template <int D, bool CAUSAL, bool SPARSE, int KG>
static void launch_dkdv(const BwdParams& p, const BwdBf16Args& a, hipStream_t stream) {
  constexpr int BK = DkvCfg<D, KG>::BK;
  const unsigned nkb = (unsigned)((p.N + BK - 1) / BK);
  // block-sparse: the list of mask rows lives in dynamic LDS
  const size_t dyn = SPARSE ? (((size_t)a.nb * 2 + 15) & ~(size_t)15) : 0;
  if (SPARSE)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, CAUSAL, SPARSE, KG>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, SPARSE, KG>), dim3(nkb * (unsigned)a.BH), dim3(128 * KG), dyn,
                     stream, a);
}

// dQ on 128-query workgroups (one per mask row when block-sparse)
template <int D, bool CAUSAL, bool SPARSE>
static void launch_dq_short(const BwdParams& p, const BwdBf16Args& a, hipStream_t stream) {
  constexpr int SBN = 32;  // keys per tile: at d = 64, three workgroups per CU
  const unsigned nqs = (unsigned)((p.N + 127) / 128);
  const size_t dyn = SPARSE ? (((size_t)a.nb * 2 + 15) & ~(size_t)15) : 0;  // the column list
  if (SPARSE)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dq_short_kernel<D, SBN, CAUSAL, SPARSE>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  hipLaunchKernelGGL((bwd_dq_short_kernel<D, SBN, CAUSAL, SPARSE>), dim3(nqs * (unsigned)a.BH), dim3(256), dyn, stream,
                     a);
}

// dQ on 256-query, 8-wave workgroups (d = 128, dense); 32-key tiles keep it within 256 VGPRs
template <int D, bool CAUSAL>
static void launch_dq_full(const BwdParams& p, const BwdBf16Args& a, hipStream_t stream) {
  const unsigned nqb = (unsigned)((p.N + 255) / 256);
  hipLaunchKernelGGL((bwd_dq_kernel<D, 32, CAUSAL>), dim3(nqb * (unsigned)a.BH), dim3(512), 0, stream, a);
}

template <int D, bool CAUSAL, bool SPARSE>
static void launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  BwdBf16Args a;
  a.q = static_cast<const unsigned short*>(p.q);
  a.k = static_cast<const unsigned short*>(p.k);
  a.v = static_cast<const unsigned short*>(p.v);
  a.dO = static_cast<const unsigned short*>(p.dO);
  a.o = static_cast<const unsigned short*>(p.o);
  a.olo = static_cast<const unsigned short*>(p.o_lo);
  a.lse = p.lse;
  a.stats = reinterpret_cast<float2*>(p.stats);
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = p.dv;
  a.grad_bf16 = p.grad_dtype == 1;
  a.BH = p.B * p.H;
  a.group = p.H / p.Hkv;
  a.N = p.N;
  a.c = fmaxf(fabsf(p.scale) * kLog2e, 0x1p-100f);
  a.scale = p.scale;
  a.neg = p.scale < 0.f ? 1 : 0;
  a.mask = p.mask;
  a.nb = (p.N + 127) / 128;
  BwdBf16Args akv = a;
  if (a.group > 1) {  // per-query-head fp32 dK / dV, summed over the groups afterwards
    akv.dk = p.part_k;
    akv.dv = p.part_v;
    akv.grad_bf16 = 0;
  }
  // the dQ kernel first: it also forms D and stores each row's (lse log2 e, -D) for the dK/dV kernel
  if constexpr (SPARSE || D == 64) {
    launch_dq_short<D, CAUSAL, SPARSE>(p, a, stream);
  } else if constexpr (CAUSAL) {
    if (p.N <= kShortCausalN) launch_dq_short<D, CAUSAL, SPARSE>(p, a, stream);
    else launch_dq_full<D, CAUSAL>(p, a, stream);
  } else {
    launch_dq_full<D, CAUSAL>(p, a, stream);
  }
  // dense d = 64 over short key ranges: 64-key workgroups, two per CU
  if constexpr (D == 64 && !SPARSE) {
    if (p.N <= (CAUSAL ? kDkvPairN : 2 * kDkvPairN)) {
      launch_dkdv<D, CAUSAL, SPARSE, 2>(p, akv, stream);
      return;
    }
  }
  launch_dkdv<D, CAUSAL, SPARSE, 4>(p, akv, stream);
}

template <int D, bool CAUSAL>
static void launch_bwd_f32(const BwdParams& p, hipStream_t stream) {
  BwdF32Args a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.dO = static_cast<const float*>(p.dO);
  a.lse = p.lse;
  a.stats = reinterpret_cast<const float2*>(p.stats);
  a.dq = static_cast<float*>(p.dq);
  const bool grouped = p.Hkv < p.H;
  a.dk = grouped ? p.part_k : static_cast<float*>(p.dk);
  a.dv = grouped ? p.part_v : static_cast<float*>(p.dv);
  a.BH = p.B * p.H;
  a.group = p.H / p.Hkv;
  a.N = p.N;
  a.scale = p.scale;
  const unsigned nk = (unsigned)((p.N + 63) / 64 * a.BH);
  hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, CAUSAL>), dim3(nk), dim3(64), 0, stream, a);
  hipLaunchKernelGGL((bwd_f32_dq_kernel<D, CAUSAL>), dim3(nk), dim3(64), 0, stream, a);
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  (void)hipGetLastError();  // clear an error left by an earlier, unrelated HIP call
  if (p.dtype == 0) {
    if (p.d == 64) {
      launch_prep_f32<64>(p, stream);
      if (p.causal) launch_bwd_f32<64, true>(p, stream); else launch_bwd_f32<64, false>(p, stream);
    } else {
      launch_prep_f32<128>(p, stream);
      if (p.causal) launch_bwd_f32<128, true>(p, stream); else launch_bwd_f32<128, false>(p, stream);
    }
    if (p.Hkv < p.H) launch_group_sum(p, stream);
    return hipGetLastError();
  }
  const bool sparse = p.mask != nullptr;
  if (p.d == 64) {
    if (sparse) {
      if (p.causal) launch_bwd_bf16<64, true, true>(p, stream); else launch_bwd_bf16<64, false, true>(p, stream);
    } else {
      if (p.causal) launch_bwd_bf16<64, true, false>(p, stream); else launch_bwd_bf16<64, false, false>(p, stream);
    }
  } else {
    if (sparse) {
      if (p.causal) launch_bwd_bf16<128, true, true>(p, stream); else launch_bwd_bf16<128, false, true>(p, stream);
    } else {
      if (p.causal) launch_bwd_bf16<128, true, false>(p, stream);
      else launch_bwd_bf16<128, false, false>(p, stream);
    }
  }
  if (p.Hkv < p.H) launch_group_sum(p, stream);
  return hipGetLastError();
}

}  // namespace fa
