// Forward kernels of exact attention for gfx950 (MI355X).
//
// Method: the FlashAttention abstract on Tri Dao's scite.ai page (IO-aware
// exact attention: tile Q, K, V so that scores live only on chip) and the
// everydayai.blog flash-attention article ("The Math Behind Flash Attention":
// softmax decomposition with a running row maximum, and the merge of partial
// softmax results; "The Flash Attention Algorithm": block sizes from on-chip
// memory, results written back to HBM once per block).
//
// bf16 kernel, one workgroup = 128 queries of one (b, h), 4 waves x 32 queries:
//   * the wave's Q rows live in VGPRs for the whole kernel (MFMA B operand);
//   * K/V tiles of BN keys stream HBM -> VGPR -> LDS, double-buffered, one
//     barrier per tile; V is transposed on the way into LDS so that P.V reads
//     16-byte key-contiguous fragments;
//   * S^T = K Q^T on bf16 MFMA puts one query per lane (16 keys per lane, the
//     other 16 in lane ^ 32), so the row max/sum is in-lane plus one exchange;
//   * online softmax in the base-2 domain, rescaling the running output only
//     when the row maximum grows by more than 2^8 (exact: the final division
//     uses the same basis);
//   * O^T += V^T P^T on bf16 MFMA, P converted to bf16 straight from the
//     accumulator registers (K rows are stored permuted so that no shuffle is
//     needed);
//   * epilogue: O = acc / l, lse = m * |scale| + ln l (natural log).
// Block-sparse: the workgroup first compacts its row of the 128x128 tile mask
// into a list of key tiles in LDS, then visits only those.
#include <math.h>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

struct FwdKernelArgs {
  const unsigned short* q;
  const unsigned short* k;
  const unsigned short* v;
  unsigned short* o;
  float* lse;
  const unsigned char* mask;
  int BH;
  int N;
  int nb;           // mask row length (ceil(N / 128))
  float c;          // |scale| * log2(e), clamped away from 0
  float scale_abs;  // |scale|
  int neg;          // scale < 0: Q is negated on load and |scale| used
};

template <int D, int BN>
struct FwdCfg {
  static constexpr int BM = 128;       // queries per workgroup
  static constexpr int THREADS = 256;  // 4 waves x 32 queries
  static constexpr int KS = D + 8;     // LDS row stride of K (elements)
  static constexpr int VS = BN + 8;    // LDS row stride of V^T
  static constexpr int KTILE = BN * KS;
  static constexpr int VTILE = D * VS;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int K_LOADS = BN * D / 8 / THREADS;  // uint4 per thread for K
  static constexpr int K_ROWS_PER_PASS = THREADS / (D / 8);
  static_assert((BN / 4) * (D / 8) == THREADS, "one V micro-block per thread");
  static_assert(K_LOADS * THREADS * 8 == BN * D, "K tile split");
};

// K and V rows of key tile kt into registers (rows past N read as zeros).
template <int D, int BN>
__device__ __forceinline__ void fwd_load_tile(BufRes kres, BufRes vres, int kt, int tid,
                                              uint4 (&kreg)[FwdCfg<D, BN>::K_LOADS], uint4 (&vreg)[4]) {
  using C = FwdCfg<D, BN>;
  const int chunk = tid % (D / 8);
  const int row0 = tid / (D / 8);
  const unsigned int tile_off = (unsigned int)kt * BN * D * 2;
#pragma unroll
  for (int p = 0; p < C::K_LOADS; ++p)
    kreg[p] = buf_load16(kres, tile_off + (unsigned int)((row0 + p * C::K_ROWS_PER_PASS) * D + chunk * 8) * 2);
  const int g = tid % (BN / 4);
  const int c = tid / (BN / 4);
#pragma unroll
  for (int r = 0; r < 4; ++r) vreg[r] = buf_load16(vres, tile_off + (unsigned int)((4 * g + r) * D + c * 8) * 2);
}

template <int D, int BN>
__device__ __forceinline__ void fwd_store_tile(unsigned short* stage, int tid,
                                               const uint4 (&kreg)[FwdCfg<D, BN>::K_LOADS],
                                               const uint4 (&vreg)[4]) {
  using C = FwdCfg<D, BN>;
  unsigned short* ks = stage;
  unsigned short* vt = stage + C::KTILE;
  const int chunk = tid % (D / 8);
  const int row0 = tid / (D / 8);
#pragma unroll
  for (int p = 0; p < C::K_LOADS; ++p) {
    const int row = row0 + p * C::K_ROWS_PER_PASS;
    *reinterpret_cast<uint4*>(ks + swap23(row) * C::KS + chunk * 8) = kreg[p];
  }
  const int g = tid % (BN / 4);
  const int c = tid / (BN / 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    *reinterpret_cast<uint2*>(vt + (c * 8 + e) * C::VS + 4 * g) = column_of(vreg, e);
  }
}

template <int D, int BN, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdKernelArgs a) {
  using C = FwdCfg<D, BN>;
  constexpr int BM = C::BM;
  constexpr int NSB = BN / 32;  // 32-key S^T blocks per tile
  constexpr int NPT = BN / 16;  // 16-key P fragments per tile
  constexpr int NDB = D / 32;   // 32-wide d blocks of the output
  __shared__ __align__(16) unsigned short smem[2 * C::STAGE];
  extern __shared__ __align__(16) unsigned short tile_list[];  // SPARSE only
  __shared__ int list_len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;
  const int nqt = (N + BM - 1) / BM;

  int qt, bh;
  if (CAUSAL) {  // longest rows first
    qt = nqt - 1 - (int)(blockIdx.x / a.BH);
    bh = (int)(blockIdx.x % a.BH);
  } else {
    qt = (int)(blockIdx.x / a.BH);
    bh = (int)(blockIdx.x % a.BH);
  }
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const unsigned int head_bytes = (unsigned int)N * D * 2;
  const BufRes qres = make_buf(a.q + hoff, head_bytes);
  const BufRes kres = make_buf(a.k + hoff, head_bytes);
  const BufRes vres = make_buf(a.v + hoff, head_bytes);
  const BufRes ores = make_buf(a.o + hoff, head_bytes);

  const int q_first = qt * BM;
  const int wave_q0 = q_first + 32 * w;
  const int qrow = wave_q0 + l32;

  // ---- which key tiles this workgroup visits
  int ntiles;
  if (SPARSE) {
    constexpr int R = 128 / BN;  // key tiles per mask column
    const unsigned char* mrow = a.mask + (size_t)qt * a.nb;
    const int ncol = CAUSAL ? min(a.nb, qt + 1) : a.nb;
    const int nkt = (N + BN - 1) / BN;
    if (w == 0) {
      int cnt = 0;
      for (int base = 0; base < ncol; base += 64) {
        const int col = base + lane;
        const bool on = col < ncol && mrow[col] != 0;
        const unsigned long long bal = __ballot(on);
        if (on) {
          const int pos = cnt + __popcll(bal & ((1ull << lane) - 1ull));
#pragma unroll
          for (int r = 0; r < R; ++r) tile_list[pos * R + r] = (unsigned short)(col * R + r);
        }
        cnt += __popcll(bal);
      }
      if (lane == 0) {
        int len = cnt * R;
        while (len > 0 && (int)tile_list[len - 1] >= nkt) --len;  // tiles past N (last column only)
        list_len = len;
      }
    }
    __syncthreads();
    ntiles = list_len;
  } else {
    const int kend = CAUSAL ? min(N, q_first + BM) : N;
    ntiles = (kend + BN - 1) / BN;
  }

  // ---- this lane's query row as MFMA B fragments (d = 16c + 8*half .. +7)
  // (the sign mask is applied unconditionally so that the loads complete here,
  // before the tile loop, and never hold up the loop's own prefetches)
  bf16x8 qf[D / 16];
  {
    const unsigned int sign = a.neg ? 0x80008000u : 0u;
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

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;
  float l_half = 0.f;
  const float c = a.c;

  uint4 kreg[C::K_LOADS];
  uint4 vreg[4];
  if (ntiles > 0) {
    const int kt0 = SPARSE ? (int)tile_list[0] : 0;
    fwd_load_tile<D, BN>(kres, vres, kt0, tid, kreg, vreg);
    fwd_store_tile<D, BN>(smem, tid, kreg, vreg);
  }

  for (int it = 0; it < ntiles; ++it) {
    const int kt = SPARSE ? (int)tile_list[it] : it;
    const bool more = it + 1 < ntiles;
    if (more) {
      const int ktn = SPARSE ? (int)tile_list[it + 1] : it + 1;
      fwd_load_tile<D, BN>(kres, vres, ktn, tid, kreg, vreg);
    }
    __syncthreads();
    const unsigned short* ks = smem + (it & 1) * C::STAGE;
    const unsigned short* vt = ks + C::KTILE;
    const int k_first = kt * BN;

    // a causal tile entirely after this wave's queries contributes nothing
    const bool skip = CAUSAL && k_first > wave_q0 + 31;
    if (!skip) {
      f32x16 s[NSB];
#pragma unroll
      for (int b = 0; b < NSB; ++b) {
        s[b] = zero16();
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
          const bf16x8 kf = lds_bf16x8(ks + (32 * b + l32) * C::KS + 16 * cc + 8 * half);
          s[b] = mfma32(kf, qf[cc], s[b]);
        }
      }
      const bool need_mask = (k_first + BN > N) || (CAUSAL && k_first + BN - 1 > wave_q0);
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < NSB; ++b) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k_first + 32 * b + acc_row_swapped(r, half);
            const bool hide = key >= N || (CAUSAL && key > qrow);
            s[b][r] = hide ? -INFINITY : s[b][r];
          }
        }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int b = 0; b < NSB; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[b][r]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      // move the basis only when the maximum grows by more than 2^8
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
      float lsum = 0.f;
#pragma unroll
      for (int b = 0; b < NSB; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[b][r], c, -mc));
          s[b][r] = p;
          lsum += p;
        }
      }
      l_half = l_half * alpha + lsum;

      bf16x8 pf[NPT];
#pragma unroll
      for (int t = 0; t < NPT; ++t) pf[t] = pack_bf16(s[t >> 1], 8 * (t & 1));
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int t = 0; t < NPT; ++t) {
          const bf16x8 vf = lds_bf16x8(vt + (32 * db + l32) * C::VS + 16 * t + 8 * half);
          oacc[db] = mfma32(vf, pf[t], oacc[db]);
        }
      }
    }
    if (more) fwd_store_tile<D, BN>(smem + ((it + 1) & 1) * C::STAGE, tid, kreg, vreg);
  }

  // ---- epilogue
  const float l = l_half + __shfl_xor(l_half, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * half;
      uint2 pk;
      pk.x = (unsigned int)float_to_bf16_bits(oacc[db][4 * i + 0] * inv) |
             ((unsigned int)float_to_bf16_bits(oacc[db][4 * i + 1] * inv) << 16);
      pk.y = (unsigned int)float_to_bf16_bits(oacc[db][4 * i + 2] * inv) |
             ((unsigned int)float_to_bf16_bits(oacc[db][4 * i + 3] * inv) << 16);
      buf_store8(ores, (unsigned int)(qrow * D + d0) * 2, pk);  // rows past N are dropped
    }
  }
  if (a.lse != nullptr && half == 0 && qrow < N) {
    a.lse[(size_t)bh * N + qrow] = l > 0.f ? m_run * a.scale_abs + logf(l) : -INFINITY;
  }
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
        kk = *reinterpret_cast<const float4*>(a.k + hoff + (size_t)key * D + col);
        vv = *reinterpret_cast<const float4*>(a.v + hoff + (size_t)key * D + col);
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
template <int D, int BN, bool CAUSAL, bool SPARSE>
static hipError_t launch_fwd_bf16_t(const FwdParams& p, hipStream_t stream) {
  FwdKernelArgs a;
  a.q = static_cast<const unsigned short*>(p.q);
  a.k = static_cast<const unsigned short*>(p.k);
  a.v = static_cast<const unsigned short*>(p.v);
  a.o = static_cast<unsigned short*>(p.o);
  a.lse = p.lse;
  a.mask = p.mask;
  a.BH = p.B * p.H;
  a.N = p.N;
  a.nb = (p.N + 127) / 128;
  const float sa = fabsf(p.scale);
  a.scale_abs = sa;
  a.c = fmaxf(sa * kLog2e, 0x1p-100f);
  a.neg = p.scale < 0.f ? 1 : 0;
  const int nqt = (p.N + 127) / 128;
  const dim3 grid((unsigned)(nqt * a.BH));
  size_t dyn = 0;
  if (SPARSE) dyn = (((size_t)a.nb * (128 / BN) * sizeof(unsigned short)) + 15) & ~(size_t)15;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, CAUSAL, SPARSE>), grid, dim3(256), dyn, stream, a);
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
  a.N = p.N;
  a.scale = p.scale;
  const int nqt = (p.N + 63) / 64;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(nqt * a.BH)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  // an error left by an earlier, unrelated HIP call must not be reported as ours
  (void)hipGetLastError();
  const bool sparse = p.mask != nullptr;
  if (p.dtype == 0) {  // fp32
    if (p.d == 64) return p.causal ? launch_fwd_f32_t<64, true>(p, stream) : launch_fwd_f32_t<64, false>(p, stream);
    return p.causal ? launch_fwd_f32_t<128, true>(p, stream) : launch_fwd_f32_t<128, false>(p, stream);
  }
  if (p.d == 64) {
    if (sparse)
      return p.causal ? launch_fwd_bf16_t<64, 128, true, true>(p, stream)
                      : launch_fwd_bf16_t<64, 128, false, true>(p, stream);
    return p.causal ? launch_fwd_bf16_t<64, 128, true, false>(p, stream)
                    : launch_fwd_bf16_t<64, 128, false, false>(p, stream);
  }
  if (sparse)
    return p.causal ? launch_fwd_bf16_t<128, 64, true, true>(p, stream)
                    : launch_fwd_bf16_t<128, 64, false, true>(p, stream);
  return p.causal ? launch_fwd_bf16_t<128, 64, true, false>(p, stream)
                  : launch_fwd_bf16_t<128, 64, false, false>(p, stream);
}

}  // namespace fa
