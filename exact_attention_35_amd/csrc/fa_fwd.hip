// Forward kernels of exact attention for gfx950 (MI355X).
//
// Method: the FlashAttention abstract on Tri Dao's scite.ai page (IO-aware
// exact attention: tile Q, K, V so that scores live only on chip) and the
// everydayai.blog flash-attention article ("The Math Behind Flash Attention":
// softmax decomposition with a running row maximum, and the merge of partial
// softmax results; "The Flash Attention Algorithm": block sizes from on-chip
// memory, results written back to HBM once per block).
//
// bf16 kernel (fwd_bf16_kernel), one workgroup = 256 queries of one (b, h),
// 8 waves x 32 queries:
//   * the wave's Q rows live in VGPRs for the whole kernel (MFMA B operand);
//   * K/V tiles of BN keys (16 KB) arrive by LDS-direct buffer loads into rings
//     of three buffers, two tiles ahead of use;
//   * S^T = K Q^T on bf16 MFMA puts one query per lane (16 keys per lane, the
//     other 16 in lane ^ 32), so the row max/sum is in-lane plus one exchange;
//     K rows sit in LDS permuted so that P converts to the next MFMA's operand
//     in registers;
//   * online softmax in the base-2 domain, rescaling the running output only
//     when the row maximum grows by more than 2^8 (exact: the final division
//     uses the same basis);
//   * O^T += V^T P^T on bf16 MFMA, V^T read with transposing LDS reads;
//   * waves w and w+4 share a SIMD and alternate MFMA and softmax phases;
//   * epilogue: O = acc / l, lse = m * |scale| + ln l (natural log).
// Grouped-query heads read K/V head bh / group.
//
// fwd_bf16_short_kernel: 128 queries and 4 waves per workgroup, two to four
// workgroups per CU, the same tiles and arithmetic.  It serves short key ranges
// (causal N <= 2048, and at d = 64 causal N <= 8192 or N <= 4096) and every
// block-sparse forward: its 128 queries are one row of the 128 x 128 tile mask,
// whose kept key tiles it lists and visits alone.
//
// fwd_f32_kernel is a plain fp32 kernel (one query per thread).
#include <math.h>

#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

namespace fa {

struct FwdKernelArgs {
  const unsigned short* q;
  const unsigned short* k;
  const unsigned short* v;
  unsigned short* o;
  unsigned short* olo;  // optional low-order part of O (null: not written)
  float* lse;
  const unsigned char* mask;
  int BH;
  int group;        // query heads per K/V head (1: plain multi-head)
  int N;
  int nb;           // mask row length (ceil(N / 128))
  float c;          // |scale| * log2(e), clamped away from 0
  float scale_abs;  // |scale|
  int neg;          // scale < 0: Q is negated on load and |scale| used
};

template <int D, int BN>
struct FwdCfg : TileCfg<D, BN> {
  static constexpr int BM = 256;      // queries per workgroup (8 waves x 32)
  static constexpr int NDB = D / 32;  // 32-wide d blocks of the output
};

// keys past N, and under causal masking keys after the query, get -inf
template <int BN, bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[BN / 32], int k_first, int qrow, int N, int half) {
#pragma unroll
  for (int b = 0; b < BN / 32; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // key = base + off with off = 16(r/8) + (r%8) a constant: compare off with per-lane bounds
      const int base = k_first + 32 * b + 8 * half;
      const int off = 16 * (r >> 3) + (r & 7);
      const bool hide = off >= N - base || (CAUSAL && off > qrow - base);
      s[b][r] = hide ? -INFINITY : s[b][r];
    }
  }
}

// row maximum of the tile for this lane's query (both half-waves); four
// independent v_max3 chains, so that one wave's dependent maxima do not stall it
template <int BN>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[BN / 32]) {
  constexpr int NE = 16 * (BN / 32);  // scores per lane: 32 or 64
  constexpr int Q = NE / 4;           // per chain: 8 or 16 (even)
  float m[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int b = c * Q;
    m[c] = max2f(s[b >> 4][b & 15], s[(b + 1) >> 4][(b + 1) & 15]);
#pragma unroll
    for (int i = 2; i < Q; i += 2)
      m[c] = max3f(m[c], s[(b + i) >> 4][(b + i) & 15], s[(b + i + 1) >> 4][(b + i + 1) & 15]);
  }
  return xhalf_max(max2f(max3f(m[0], m[1], m[2]), m[3]));
}

// P~ = exp2(S c - m c) -> bf16 MFMA fragments; returns the fp32 row sum of this half-wave
template <int BN>
__device__ __forceinline__ float exp_tile(const f32x16 (&s)[BN / 32], float c, float mc, bf16x8 (&pf)[BN / 16]) {
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: no serial add chain
#pragma unroll
  for (int t = 0; t < BN / 16; ++t) {
    bf16x8 frag;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + e], c, -mc));
      lsum[e & 3] += p;
      frag[e] = (__bf16)p;
    }
    pf[t] = frag;
  }
  return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
}

// Schedule of one MFMA phase: LDS fragment reads run ahead of the MFMAs
// (masks: 0x8 MFMA, 0x100 LDS read).  P.V takes two reads per MFMA, S^T one.
template <int D, int BN>
__device__ __forceinline__ void sched_gemm_phase() {
  constexpr int NPV = (BN / 16) * (D / 32);
  constexpr int NQK = (BN / 32) * (D / 16);
#pragma unroll
  for (int i = 0; i < 6; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int i = 0; i < NPV - 3; ++i) {
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

// this lane's query row as MFMA B fragments (d = 16c + 8*half .. +7); a negative
// scale is carried by negating Q on load
template <int D>
__device__ __forceinline__ void load_q_frags(BufRes qres, int qrow, int half, int neg, bf16x8 (&qf)[D / 16]) {
  const unsigned int sign = neg ? 0x80008000u : 0u;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    uint4 u = buf_load16(qres, (unsigned int)(qrow * D + 16 * c + 8 * half) * 2);
    u.x ^= sign;
    u.y ^= sign;
    u.z ^= sign;
    u.w ^= sign;
    qf[c] = as_bf16x8(u);
  }
}

// Online-softmax step for one score tile: row maximum, P = exp2(S c - m c) and the
// running half-row sum.  The basis m moves only when the maximum grows by more than
// 2^8, and the running output is rescaled then (exact: the final division uses the
// same basis).
template <int BN, int NDB>
__device__ __forceinline__ void softmax_update(const f32x16 (&s)[BN / 32], float c, float& m_run, float& l_half,
                                               f32x16 (&oacc)[NDB], bf16x8 (&pf)[BN / 16]) {
  const float mt = tile_max<BN>(s);
  const bool grow = (mt - m_run) * c > 8.f;
  float alpha = 1.f;
  if (grow) {
    alpha = __builtin_amdgcn_exp2f((m_run - mt) * c);
    m_run = mt;
  }
  if (__ballot(grow)) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
  }
  const float mc = m_run == -INFINITY ? 0.f : m_run * c;
  l_half = l_half * alpha + exp_tile<BN>(s, c, mc, pf);
}

// Epilogue for this lane's query row: O = acc / l in bf16 through ores; when olo (the
// head's low-order output) is given, also bf16(O - fp32(bf16(O))), so that the two
// together carry O to about 16 significant bits; when lse (the head's row) is given,
// lse = m |scale| + ln l.  Rows past N are dropped by the range-checked stores.
template <int D>
__device__ __forceinline__ void store_output(const f32x16 (&oacc)[D / 32], float m_run, float l_half, BufRes ores,
                                             unsigned short* olo, float* lse, float scale_abs, int N,
                                             unsigned int head_bytes, int qrow, int half) {
  const float l = xhalf_sum(l_half);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const bool want_lo = olo != nullptr;
  const BufRes lores = make_buf(olo, head_bytes);  // used only when want_lo
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * half;
      unsigned short hb[4], lb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = oacc[db][4 * i + e] * inv;
        hb[e] = float_to_bf16_bits(x);
        lb[e] = float_to_bf16_bits(x - bf16_bits_to_float(hb[e]));  // exact difference, then rounded
      }
      const uint2 pk = make_uint2((unsigned int)hb[0] | ((unsigned int)hb[1] << 16),
                                  (unsigned int)hb[2] | ((unsigned int)hb[3] << 16));
      buf_store8(ores, (unsigned int)(qrow * D + d0) * 2, pk);
      if (want_lo) {
        const uint2 pl = make_uint2((unsigned int)lb[0] | ((unsigned int)lb[1] << 16),
                                    (unsigned int)lb[2] | ((unsigned int)lb[3] << 16));
        buf_store8(lores, (unsigned int)(qrow * D + d0) * 2, pl);
      }
    }
  }
  if (lse != nullptr && half == 0 && qrow < N) {
    lse[qrow] = l > 0.f ? m_run * scale_abs + logf(l) : -INFINITY;
  }
}

// Forward kernel: one workgroup = 256 queries of one (b, h), 8 waves of 32 queries.
// Waves w and w+4 share a SIMD and form two groups (A = waves 0-3, B = 4-7) that
// alternate between an MFMA phase G(t) = {O += V(t-1) P(t-1), S(t) = K(t) Q^T} and
// a VALU phase S(t) = {row max, rescale, P(t) = exp2(S c - m c)}: while one group
// issues MFMAs the other one's softmax runs on the vector ALU of the same SIMD.
// The MFMA phase runs at raised wave priority so that its MFMAs issue first.
// Tiles arrive by LDS-direct loads into a ring of three buffers, two steps
// ahead of their use (group A fetches V, group B fetches K).  (Block-sparse
// forwards run on fwd_bf16_short_kernel, whose 128 queries are one mask row.)
template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(512) void fwd_bf16_kernel(FwdKernelArgs a) {
  using C = FwdCfg<D, BN>;
  constexpr int BM = C::BM;
  constexpr int NSB = C::NSB;
  constexpr int NPT = C::NPT;
  constexpr int NDB = C::NDB;
  constexpr int NW = 4;                         // waves of a group that load one tile
  constexpr int LPW = C::TILE * 2 / 1024 / NW;  // 1 KB loads per wave per tile
  // separate arrays (not one): the compiler then knows that LDS reads of one
  // buffer do not depend on LDS-direct loads still landing in another
  __shared__ __align__(16) unsigned short kbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short kbuf_1[C::TILE];
  __shared__ __align__(16) unsigned short kbuf_2[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_1[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_2[C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int grp = w >> 2;  // 0: group A, 1: group B
  const int wg = w & 3;    // wave index inside the group (= SIMD)
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
  const BufRes ores = make_buf(a.o + hoff, head_bytes);

  const int q_first = qt * BM;
  // query blocks interleave between the groups so that causal work is balanced
  const int wave_q0 = q_first + 32 * (2 * wg + grp);
  const int qrow = wave_q0 + l32;
  // this wave's share of a tile load, made wave-uniform so that the loads' LDS
  // destinations (M0) are formed in scalar registers rather than read out of VGPRs
  const int wi = __builtin_amdgcn_readfirstlane(wg);
  unsigned short* const kb0 = kbuf_0;
  unsigned short* const kb1 = kbuf_1;
  unsigned short* const kb2 = kbuf_2;
  unsigned short* const vb0 = vbuf_0;
  unsigned short* const vb1 = vbuf_1;
  unsigned short* const vb2 = vbuf_2;

  // ---- the key tiles this workgroup visits
  const int kend = CAUSAL ? min(N, q_first + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  const int nsteps = ntiles;
  auto tile_at = [&](int t) __attribute__((always_inline)) -> int {  // steps past the end repeat the last tile
    return min(t, ntiles - 1);
  };
  auto need_mask = [&](int kt) __attribute__((always_inline)) -> bool {
    const int k_first = kt * BN;
    return (k_first + BN > N) || (CAUSAL && k_first + BN - 1 > wave_q0);
  };

  bf16x8 qf[D / 16];
  load_q_frags<D>(qres, qrow, half, a.neg, qf);
  const KOffsets<D> ko = k_offsets<D>(l32, half);
  const VOffsets<D> vo = v_offsets<D>(lane);

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;
  float l_half = 0.f;
  const float c = a.c;
  f32x16 s[NSB];
  bf16x8 pf[NPT];
#pragma unroll
  for (int b = 0; b < NSB; ++b) s[b] = zero16();
#pragma unroll
  for (int t = 0; t < NPT; ++t) pf[t] = as_bf16x8(zero_uint4());

  // V buffers start as zeros: the first MFMA phase multiplies buffer 2 by P = 0,
  // and key rows past N (which the range-checked loads may leave unwritten) must
  // hold finite values, since they are multiplied by P = 0 as well
  for (int i = tid; i < C::TILE / 8; i += 512) {
    reinterpret_cast<uint4*>(vbuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_1)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_2)[i] = zero_uint4();
  }
  barrier_lds();
  if (ntiles > 0) {
    if (grp == 1) {
      dma_k<D, BN, NW>(kres, kb0, tile_at(0), wi, lane);
      dma_k<D, BN, NW>(kres, kb1, tile_at(1), wi, lane);
    } else {
      dma_v<D, BN, NW>(vres, vb0, tile_at(0), wi, lane);
      wait_dma();
    }
  }
  barrier_ring<LPW>();  // K(1) may still be landing

  // Branch-free so that the LDS reads run ahead of the MFMAs: at t = 0 the P.V
  // product uses P = 0 and at t = ntiles the S^T of a stale tile is never used.
  auto gemm_phase = [&](int t, const unsigned short* kcur, const unsigned short* vprev) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    pv_tile<D, BN>(vprev, vo, pf, oacc);
    qk_tile<D, BN>(kcur, ko, qf, s);
    sched_gemm_phase<D, BN>();
    if (t < ntiles) {
      const int kt = tile_at(t);
      if (need_mask(kt)) {
        mask_tile<BN, CAUSAL>(s, kt * BN, qrow, N, half);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // S(t): softmax statistics and P(t) = exp2(S c - m c)
  auto softmax_phase = [&]() __attribute__((always_inline)) { softmax_update<BN, NDB>(s, c, m_run, l_half, oacc, pf); };

  // Step t.  Buffers rotate with t mod 3: kcur holds K(t), vprev V(t-1); at the
  // top of its MFMA phase group A starts fetching V(t+1) into vnext and group B
  // K(t+2) into knext2 (steps past the end fetch the last tile again, so every
  // step issues the same number of loads).  At the end of the step each wave
  // waits for the loads it issued one step earlier, which the next step reads.
  auto step = [&](int t, const unsigned short* kcur, unsigned short* knext2, const unsigned short* vprev,
                  unsigned short* vnext) __attribute__((always_inline)) {
    // phase 2t: A fetches V(t+1) and runs G(t); B runs S(t-1).  Each group issues
    // its tile loads in its MFMA phase, where they cost nothing: issued next to
    // the vector work of a softmax phase they would slow it down.
    const bool active = ntiles > 0 && t <= ntiles;
    if (grp == 0) {
      if (active) {
        dma_v<D, BN, NW>(vres, vnext, tile_at(t + 1), wi, lane);
        gemm_phase(t, kcur, vprev);
      }
    } else {
      if (t >= 1 && t - 1 < ntiles) softmax_phase();
    }
    barrier_plain();
    // phase 2t+1: A runs S(t); B fetches K(t+2) and runs G(t)
    if (grp == 0) {
      if (t < ntiles) softmax_phase();
    } else {
      if (active) {
        dma_k<D, BN, NW>(kres, knext2, tile_at(t + 2), wi, lane);
        gemm_phase(t, kcur, vprev);
      }
    }
    barrier_ring<LPW>();
  };
  // every wave runs the same steps (the barriers need it)
  for (int t = 0; nsteps > 0 && t <= nsteps; t += 3) {
    step(t, kb0, kb2, vb2, vb1);
    if (t + 1 <= nsteps) step(t + 1, kb1, kb0, vb0, vb2);
    if (t + 2 <= nsteps) step(t + 2, kb2, kb1, vb1, vb0);
  }
  wait_dma();  // no LDS-direct load may outlive the workgroup

  store_output<D>(oacc, m_run, l_half, ores, a.olo ? a.olo + hoff : nullptr, a.lse ? a.lse + (size_t)bh * N : nullptr,
                  a.scale_abs, N, head_bytes, qrow, half);
}

// Forward kernel for short causal sequences: one workgroup = 128 queries of one
// (b, h), 4 waves of 32 queries, one wave per SIMD.  Each wave runs its own MFMA
// phase G(t) and softmax phase S(t) in turn (the same tiles, fragments and
// arithmetic as fwd_bf16_kernel, so the results are the same bit for bit).  Tiles
// go through rings of two LDS buffers, one step ahead: step t fetches K(t+1) and
// V(t) while it computes O += V(t-1) P(t-1), S(t) = K(t) Q^T and the softmax of
// tile t.  With 64 KB of LDS two workgroups share a CU, so one's prologue,
// pipeline fill and epilogue overlap the other's steady state: over a short key
// range these fixed costs, and the wasted half of the diagonal tile under causal
// masking, outweigh the MFMA/softmax overlap of the 8-wave kernel.  With 64-key
// tiles at d = 64 (32 KB of LDS) the kernel is held to 128 registers, so that four
// workgroups share a CU; with 32-key tiles at d = 128 (32 KB) to 168, three per CU.
template <int D, int BN, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 && BN == 64 ? 4 : (D == 128 && BN == 32 ? 3 : 1), 8)))
void fwd_bf16_short_kernel(FwdKernelArgs a) {
  using C = FwdCfg<D, BN>;
  constexpr int BM = 128;
  constexpr int NSB = C::NSB;
  constexpr int NPT = C::NPT;
  constexpr int NDB = C::NDB;
  __shared__ __align__(16) unsigned short kbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short kbuf_1[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_0[C::TILE];
  __shared__ __align__(16) unsigned short vbuf_1[C::TILE];
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
  const GridPos gp = (CAUSAL && !SPARSE) ? grid_pos_causal(nqt, a.BH, 32 * (D == 64 && BN == 64 ? 4 : (D == 128 && BN == 32 ? 3 : 2)))
                                         : grid_pos<HR>(nqt, a.BH);
  const int qt = CAUSAL ? nqt - 1 - gp.r : gp.r;  // longest rows first
  const int bh = gp.bh;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const size_t kvoff = (size_t)(bh / a.group) * (size_t)N * D;  // grouped-query: shared K/V head
  const unsigned int head_bytes = (unsigned int)N * D * 2;
  const BufRes qres = make_buf(a.q + hoff, head_bytes);
  const BufRes kres = make_buf(a.k + kvoff, head_bytes);
  const BufRes vres = make_buf(a.v + kvoff, head_bytes);
  const BufRes ores = make_buf(a.o + hoff, head_bytes);

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

  bf16x8 qf[D / 16];
  load_q_frags<D>(qres, qrow, half, a.neg, qf);
  const KOffsets<D> ko = k_offsets<D>(l32, half);
  const VOffsets<D> vo = v_offsets<D>(lane);
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;
  float l_half = 0.f;
  const float c = a.c;
  f32x16 s[NSB];
  bf16x8 pf[NPT];
#pragma unroll
  for (int b = 0; b < NSB; ++b) s[b] = zero16();
#pragma unroll
  for (int t = 0; t < NPT; ++t) pf[t] = as_bf16x8(zero_uint4());

  // V buffers start as zeros: step 0 multiplies buffer 1 by P = 0, and key rows
  // past N (which the range-checked loads may leave unwritten) must hold finite
  // values, since they are multiplied by P = 0 as well
  for (int i = tid; i < C::TILE / 8; i += 256) {
    reinterpret_cast<uint4*>(vbuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_1)[i] = zero_uint4();
  }
  barrier_lds();
  if (ntiles > 0) dma_k<D, BN, 4>(kres, kbuf_0, tile_at(0), wi, lane);
  barrier_ring<0>();  // K(0) has landed

  // step t: buffers alternate with t mod 2 (kcur holds K(t), vprev V(t-1)); the
  // loads it issues land by the barrier that ends it.  At t = 0 the P.V product
  // uses P = 0; at t = ntiles the S^T of a repeated tile is never used.
  auto step = [&](int t, const unsigned short* kcur, unsigned short* knext, const unsigned short* vprev,
                  unsigned short* vcur) __attribute__((always_inline)) {
    dma_k<D, BN, 4>(kres, knext, tile_at(t + 1), wi, lane);
    dma_v<D, BN, 4>(vres, vcur, tile_at(t), wi, lane);
    pv_tile<D, BN>(vprev, vo, pf, oacc);
    qk_tile<D, BN>(kcur, ko, qf, s);
    sched_gemm_phase<D, BN>();
    if (t < ntiles) {
      const int kt = tile_at(t);
      if (need_mask(kt)) mask_tile<BN, CAUSAL>(s, kt * BN, qrow, N, half);
      softmax_update<BN, NDB>(s, c, m_run, l_half, oacc, pf);
    }
    barrier_ring<0>();
  };
  // a block-sparse row without any kept tile stays inactive: O = 0 and lse = -inf
  for (int t = 0; ntiles > 0 && t <= ntiles; t += 2) {
    step(t, kbuf_0, kbuf_1, vbuf_1, vbuf_0);
    if (t + 1 <= ntiles) step(t + 1, kbuf_1, kbuf_0, vbuf_0, vbuf_1);
  }
  wait_dma();  // no LDS-direct load may outlive the workgroup

  store_output<D>(oacc, m_run, l_half, ores, a.olo ? a.olo + hoff : nullptr, a.lse ? a.lse + (size_t)bh * N : nullptr,
                  a.scale_abs, N, head_bytes, qrow, half);
}

// ---------------------------------------------------------------------------
// fp32 forward: a plain correctness kernel (one query per thread, keys staged
// through LDS 32 at a time, online softmax per key).  Not tuned.
// ---------------------------------------------------------------------------
struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int BH;
  int group;
  int N;
  float scale;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdF32Args a) {
  constexpr int BM = 64;
  constexpr int BN = 32;
  __shared__ __align__(16) float ks[BN * D];
  __shared__ __align__(16) float vs[BN * D];
  const int tid = threadIdx.x;
  const int N = a.N;
  const int nqt = (N + BM - 1) / BM;
  const int qt = (int)(blockIdx.x / a.BH);
  const int bh = (int)(blockIdx.x % a.BH);
  (void)nqt;
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(bh / a.group) * N * D;
  const int qrow = qt * BM + tid;
  const bool in = qrow < N;
  float qv[D];
  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qv[i] = in ? a.q[hoff + (size_t)qrow * D + i] : 0.f;
    acc[i] = 0.f;
  }
  float m = -INFINITY;
  float l = 0.f;
  const int kend = CAUSAL ? min(N, qt * BM + BM) : N;
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int idx = tid; idx < BN * D / 4; idx += 64) {
      const int row = idx / (D / 4);
      const int col = (idx % (D / 4)) * 4;
      const int key = k0 + row;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (key < N) {
        kk = *reinterpret_cast<const float4*>(a.k + kvoff + (size_t)key * D + col);
        vv = *reinterpret_cast<const float4*>(a.v + kvoff + (size_t)key * D + col);
      }
      *reinterpret_cast<float4*>(ks + row * D + col) = kk;
      *reinterpret_cast<float4*>(vs + row * D + col) = vv;
    }
    __syncthreads();
    const int jn = min(BN, kend - k0);
    for (int j = 0; j < jn; ++j) {
      const int key = k0 + j;
      if (CAUSAL && key > qrow) break;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) dot = fmaf(qv[i], ks[j * D + i], dot);
      const float s = dot * a.scale;
      if (s > m) {
        const float alpha = m == -INFINITY ? 0.f : expf(m - s);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] *= alpha;
        m = s;
      }
      const float p = expf(s - m);
      l += p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(p, vs[j * D + i], acc[i]);
    }
  }
  if (in) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < D; i += 4) {
      *reinterpret_cast<float4*>(a.o + hoff + (size_t)qrow * D + i) =
          make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
    }
    if (a.lse) a.lse[(size_t)bh * N + qrow] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static FwdKernelArgs fwd_args(const FwdParams& p) {
  FwdKernelArgs a;
  a.q = static_cast<const unsigned short*>(p.q);
  a.k = static_cast<const unsigned short*>(p.k);
  a.v = static_cast<const unsigned short*>(p.v);
  a.o = static_cast<unsigned short*>(p.o);
  a.olo = static_cast<unsigned short*>(p.o_lo);
  a.lse = p.lse;
  a.mask = p.mask;
  a.BH = p.B * p.H;
  a.group = p.H / p.Hkv;
  a.N = p.N;
  a.nb = (p.N + 127) / 128;
  const float sa = fabsf(p.scale);
  a.scale_abs = sa;
  a.c = fmaxf(sa * kLog2e, 0x1p-100f);
  a.neg = p.scale < 0.f ? 1 : 0;
  return a;
}

template <int D, int BN, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const FwdParams& p, hipStream_t stream) {
  const FwdKernelArgs a = fwd_args(p);
  const int nqt = (p.N + 255) / 256;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, CAUSAL>), dim3((unsigned)(nqt * a.BH)), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BN, bool CAUSAL, bool SPARSE = false>
static hipError_t launch_fwd_short_t(const FwdParams& p, hipStream_t stream) {
  const FwdKernelArgs a = fwd_args(p);
  const int nqt = (p.N + 127) / 128;
  // block-sparse: the column list lives in dynamic LDS next to the static tiles
  const size_t dyn = SPARSE ? (((size_t)a.nb * sizeof(unsigned short)) + 15) & ~(size_t)15 : 0;
  if (SPARSE)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_bf16_short_kernel<D, BN, CAUSAL, SPARSE>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  hipLaunchKernelGGL((fwd_bf16_short_kernel<D, BN, CAUSAL, SPARSE>), dim3((unsigned)(nqt * a.BH)), dim3(256), dyn,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_f32_t(const FwdParams& p, hipStream_t stream) {
  FwdF32Args a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<float*>(p.o);
  a.lse = p.lse;
  a.BH = p.B * p.H;
  a.group = p.H / p.Hkv;
  a.N = p.N;
  a.scale = p.scale;
  const int nqt = (p.N + 63) / 64;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(nqt * a.BH)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

// When fwd_bf16_short_kernel serves a dense bf16 forward (measured on MI355X, bf16,
// 12-16 heads, against fwd_bf16_kernel, interleaved on one box):
//  * d = 64, 64-key tiles, four workgroups per CU: causal N <= 8192 on grids of at
//    least 512 workgroups (21-37% faster at N = 512-2048, 15% at 4096, 4% at 8192;
//    1-3% slower from 16K on); without causal masking N <= 4096 on any grid (6-23%
//    faster, 17-20% on grids of 256 workgroups; 3% slower at 16K-32K);
//  * d = 64, 128-key tiles, two per CU: causal N <= 2048 on smaller grids (21% faster
//    on 256 workgroups, where the 64-key tiles were 8% slower still: the CUs cannot be
//    filled either way and the shorter tiles only add steps);
//  * d = 128, 32-key tiles, three per CU: causal N <= 2048 (9-16% faster, 23% on a grid
//    of 128 workgroups; even at N = 4096); without causal masking 3-20% slower.
constexpr int kShortCausalN = 2048;
constexpr int kShortD64CausalN = 8192;
constexpr int kShortD64N = 4096;
constexpr long long kShortSmallTileGrid = 512;

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  // an error left by an earlier, unrelated HIP call must not be reported as ours
  (void)hipGetLastError();
  const bool sparse = p.mask != nullptr;
  if (p.dtype == 0) {  // fp32
    if (p.d == 64) return p.causal ? launch_fwd_f32_t<64, true>(p, stream) : launch_fwd_f32_t<64, false>(p, stream);
    return p.causal ? launch_fwd_f32_t<128, true>(p, stream) : launch_fwd_f32_t<128, false>(p, stream);
  }
  // block-sparse: one 128-query workgroup per mask row
  if (sparse) {
    if (p.d == 64)
      return p.causal ? launch_fwd_short_t<64, 64, true, true>(p, stream) : launch_fwd_short_t<64, 64, false, true>(p, stream);
    return p.causal ? launch_fwd_short_t<128, 32, true, true>(p, stream) : launch_fwd_short_t<128, 32, false, true>(p, stream);
  }
  // short key ranges: 128-query, 4-wave workgroups, several per CU
  const long long nwg = (long long)((p.N + 127) / 128) * p.B * p.H;
  if (p.d == 64) {
    if (p.causal ? (p.N <= kShortD64CausalN && nwg >= kShortSmallTileGrid) : p.N <= kShortD64N)
      return p.causal ? launch_fwd_short_t<64, 64, true>(p, stream) : launch_fwd_short_t<64, 64, false>(p, stream);
    if (p.causal && p.N <= kShortCausalN) return launch_fwd_short_t<64, 128, true>(p, stream);
    return p.causal ? launch_fwd_bf16_t<64, 128, true>(p, stream) : launch_fwd_bf16_t<64, 128, false>(p, stream);
  }
  if (p.causal && p.N <= kShortCausalN) return launch_fwd_short_t<128, 32, true>(p, stream);
  return p.causal ? launch_fwd_bf16_t<128, 64, true>(p, stream) : launch_fwd_bf16_t<128, 64, false>(p, stream);
}

}  // namespace fa
