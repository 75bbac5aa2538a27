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
// bf16 kernel: one workgroup owns 128 keys of one (b, h) (4 waves x 32 keys);
// its K and V rows stay in VGPRs (MFMA B operands) and dK, dV accumulate in
// registers.  It walks the query tiles (64 rows; under causal masking only
// those at or after its keys), staging Q and dO through LDS both row-major and
// transposed.  Per wave and 32-query block: S = Q K^T and dP = dO V^T on MFMA
// (one key per lane), P = exp2(S c - lse log2 e), dS = P (dP - D), then
// dV += P^T dO and dK += dS^T Q from the registers.  dS goes through LDS so
// that the workgroup computes dQ_i = dS K over all its 128 keys and adds it to
// an fp32 accumulator with atomics.
#include <math.h>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// D = rowsum(dO * O), fp32 out.  T = unsigned short (bf16 bits) or float.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* __restrict__ o, const T* __restrict__ dO,
                                                        float* __restrict__ delta, long long rows) {
  constexpr int EPT = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int TPR = D / EPT;         // threads per row
  constexpr int RPB = 256 / TPR;       // rows per block
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int part = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 ov = *reinterpret_cast<const uint4*>(o + row * D + part * EPT);
    const uint4 dv = *reinterpret_cast<const uint4*>(dO + row * D + part * EPT);
    if (sizeof(T) == 2) {
      const unsigned short* a = reinterpret_cast<const unsigned short*>(&ov);
      const unsigned short* b = reinterpret_cast<const unsigned short*>(&dv);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(bf16_bits_to_float(a[e]), bf16_bits_to_float(b[e]), acc);
    } else {
      const float* a = reinterpret_cast<const float*>(&ov);
      const float* b = reinterpret_cast<const float*>(&dv);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(a[e], b[e], acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) delta[row] = acc;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* __restrict__ p, long long n4) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float4* __restrict__ src,
                                                          uint2* __restrict__ dst, long long n4) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) {
    const float4 x = src[i];
    uint2 r;
    r.x = (unsigned int)float_to_bf16_bits(x.x) | ((unsigned int)float_to_bf16_bits(x.y) << 16);
    r.y = (unsigned int)float_to_bf16_bits(x.z) | ((unsigned int)float_to_bf16_bits(x.w) << 16);
    dst[i] = r;
  }
}

// ---------------------------------------------------------------------------
// bf16 main backward kernel
// ---------------------------------------------------------------------------
struct BwdKernelArgs {
  const unsigned short* q;
  const unsigned short* k;
  const unsigned short* v;
  const unsigned short* dO;
  const float* lse;
  const float* delta;
  float* dq_acc;
  void* dk;
  void* dv;
  int grad_bf16;
  int BH;
  int N;
  float c;          // |scale| * log2(e), clamped away from 0
  float scale_abs;  // factor of dK (Q is negated when scale < 0)
  float scale;      // factor of dQ
  int neg;
};

template <int D>
struct BwdCfg {
  static constexpr int BN = 128;  // keys per workgroup
  static constexpr int BM = 64;   // queries per step
  static constexpr int THREADS = 256;
  static constexpr int RS = D + 8;    // row-major Q / dO stride
  static constexpr int TS = BM + 8;   // transposed Q / dO stride
  static constexpr int KTS = BN + 8;  // transposed K stride
  static constexpr int SS = BN + 8;   // dS stride
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + BM * RS;
  static constexpr int OFF_QT = OFF_DO + BM * RS;
  static constexpr int OFF_DOT = OFF_QT + D * TS;
  static constexpr int OFF_KT = OFF_DOT + D * TS;
  static constexpr int OFF_DS = OFF_KT + D * KTS;
  static constexpr int ELEMS = OFF_DS + BM * SS;  // unsigned short elements
  static constexpr int MB_PER_TENSOR = (BM / 4) * (D / 8);  // 4x8 micro-blocks per Q (or dO) tile
  static constexpr int MB_PER_THREAD = 2 * MB_PER_TENSOR / THREADS;  // Q and dO together
  static_assert(MB_PER_THREAD * THREADS == 2 * MB_PER_TENSOR, "micro-block split");
};

// Stage one 4-row x 8-column micro-block both row-major (rows stored with
// swap23 inside 32-row groups) and transposed.
template <int RS, int TS>
__device__ __forceinline__ void stage_micro_block(unsigned short* rowmajor, unsigned short* transposed,
                                                  const uint4 (&rows)[4], int g, int c) {
#pragma unroll
  for (int r = 0; r < 4; ++r) *reinterpret_cast<uint4*>(rowmajor + swap23(4 * g + r) * RS + 8 * c) = rows[r];
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<uint2*>(transposed + (8 * c + e) * TS + 4 * g) = column_of(rows, e);
}

template <int D>
struct QTileRegs {
  uint4 mb[BwdCfg<D>::MB_PER_THREAD][4];
  float stat;
};

template <int D>
__device__ __forceinline__ void bwd_load_qtile(const BwdKernelArgs& a, BufRes qres, BufRes dores, size_t hoff,
                                               int q0, int tid, QTileRegs<D>& t) {
  using C = BwdCfg<D>;
  const int N = a.N;
#pragma unroll
  for (int j = 0; j < C::MB_PER_THREAD; ++j) {
    const int mb = tid + j * C::THREADS;  // [0, MB_PER_TENSOR) -> Q, the rest -> dO (wave-uniform)
    const bool isq = mb < C::MB_PER_TENSOR;
    const int m = isq ? mb : mb - C::MB_PER_TENSOR;
    const int g = m % (C::BM / 4);
    const int c = m / (C::BM / 4);
    const BufRes res = isq ? qres : dores;
    const unsigned int sign = (isq && a.neg) ? 0x80008000u : 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint4 u = buf_load16(res, (unsigned int)((q0 + 4 * g + r) * D + 8 * c) * 2);  // rows past N: zeros
      u.x ^= sign;
      u.y ^= sign;
      u.z ^= sign;
      u.w ^= sign;
      t.mb[j][r] = u;
    }
  }
  t.stat = 0.f;
  if (tid < 2 * C::BM) {
    const int i = tid % C::BM;
    const int row = q0 + i;
    const size_t idx = hoff / D + (size_t)row;
    if (tid < C::BM) {
      // P = exp2(S c - lse log2 e); a row past N or with no visible key gets +inf so that P = 0
      float x = INFINITY;
      if (row < N) {
        const float l = a.lse[idx];
        x = l == -INFINITY ? INFINITY : l * kLog2e;
      }
      t.stat = x;
    } else {
      t.stat = row < N ? a.delta[idx] : 0.f;
    }
  }
}

template <int D>
__device__ __forceinline__ void bwd_store_qtile(unsigned short* smem, float* lse2, float* dlt, int tid,
                                                const QTileRegs<D>& t) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int j = 0; j < C::MB_PER_THREAD; ++j) {
    const int mb = tid + j * C::THREADS;
    const bool isq = mb < C::MB_PER_TENSOR;
    const int m = isq ? mb : mb - C::MB_PER_TENSOR;
    const int g = m % (C::BM / 4);
    const int c = m / (C::BM / 4);
    stage_micro_block<C::RS, C::TS>(smem + (isq ? C::OFF_Q : C::OFF_DO), smem + (isq ? C::OFF_QT : C::OFF_DOT),
                                    t.mb[j], g, c);
  }
  if (tid < C::BM) {
    lse2[tid] = t.stat;
  } else if (tid < 2 * C::BM) {
    dlt[tid - C::BM] = t.stat;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(BwdKernelArgs a) {
  using C = BwdCfg<D>;
  constexpr int BN = C::BN;
  constexpr int BM = C::BM;
  constexpr int NDB = D / 32;
  __shared__ __align__(16) unsigned short smem[C::ELEMS];
  __shared__ __align__(16) float lse2[BM];
  __shared__ __align__(16) float dlt[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;
  const int nkt = (N + BN - 1) / BN;
  (void)nkt;
  const int kt = (int)(blockIdx.x / a.BH);  // causal: small kt = most query tiles, launched first
  const int bh = (int)(blockIdx.x % a.BH);
  const size_t hoff = (size_t)bh * N * D;
  const unsigned int head_bytes = (unsigned int)N * D * 2;
  const BufRes qres = make_buf(a.q + hoff, head_bytes);
  const BufRes kres = make_buf(a.k + hoff, head_bytes);
  const BufRes vres = make_buf(a.v + hoff, head_bytes);
  const BufRes dores = make_buf(a.dO + hoff, head_bytes);
  const int k0 = kt * BN;
  const int wave_k0 = k0 + 32 * w;
  const int mykey = wave_k0 + l32;

  // K, V rows of this lane's key as MFMA B fragments (d = 16c + 8*half .. +7)
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const unsigned int off = (unsigned int)(mykey * D + 16 * c + 8 * half) * 2;  // keys past N: zeros
    kf[c] = as_bf16x8(buf_load16(kres, off));
    vf[c] = as_bf16x8(buf_load16(vres, off));
  }
  // K^T of the workgroup's 128 keys in LDS, for dQ = dS K
  {
    constexpr int MBK = (BN / 4) * (D / 8);
    for (int m = tid; m < MBK; m += C::THREADS) {
      const int g = m % (BN / 4);
      const int c = m / (BN / 4);
      uint4 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) rows[r] = buf_load16(kres, (unsigned int)((k0 + 4 * g + r) * D + 8 * c) * 2);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint2*>(smem + C::OFF_KT + (8 * c + e) * C::KTS + 4 * g) = column_of(rows, e);
    }
  }

  f32x16 dv_acc[NDB], dk_acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dv_acc[i] = zero16();
    dk_acc[i] = zero16();
  }
  const float c = a.c;
  const int nqt = (N + BM - 1) / BM;
  const int qt_first = CAUSAL ? k0 / BM : 0;

  QTileRegs<D> regs;
  if (qt_first < nqt) {
    bwd_load_qtile<D>(a, qres, dores, hoff, qt_first * BM, tid, regs);
    bwd_store_qtile<D>(smem, lse2, dlt, tid, regs);
  }

  for (int it = qt_first; it < nqt; ++it) {
    const int q0 = it * BM;
    const bool more = it + 1 < nqt;
    __syncthreads();  // tile `it` staged; previous dS reads finished
    if (more) bwd_load_qtile<D>(a, qres, dores, hoff, q0 + BM, tid, regs);

#pragma unroll
    for (int qb = 0; qb < BM / 32; ++qb) {
      const int qb0 = q0 + 32 * qb;
      unsigned short* ds_out = smem + C::OFF_DS + (32 * qb) * C::SS + 32 * w + l32;
      // every key of this wave after every query of the block: P = 0
      if (CAUSAL && wave_k0 > qb0 + 31) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ds_out[acc_row_swapped(r, half) * C::SS] = 0;
        continue;
      }
      f32x16 s = zero16(), dp = zero16();
      const unsigned short* qrow = smem + C::OFF_Q + (32 * qb + l32) * C::RS + 8 * half;
      const unsigned short* dorow = smem + C::OFF_DO + (32 * qb + l32) * C::RS + 8 * half;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        s = mfma32(lds_bf16x8(qrow + 16 * cc), kf[cc], s);
        dp = mfma32(lds_bf16x8(dorow + 16 * cc), vf[cc], dp);
      }
      // per-register query statistics: queries 32qb + 8*half + {0..7} and +16
      float st_l[16], st_d[16];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int base = 32 * qb + 16 * hh + 8 * half;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse2 + base);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse2 + base + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(dlt + base);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(dlt + base + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st_l[8 * hh + e] = l0[e];
          st_l[8 * hh + 4 + e] = l1[e];
          st_d[8 * hh + e] = d0[e];
          st_d[8 * hh + 4 + e] = d1[e];
        }
      }
      const bool need_mask = (k0 + 32 * w + 31 >= N) || (CAUSAL && wave_k0 + 31 > qb0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -st_l[r]));
        if (need_mask) {
          const int qidx = qb0 + acc_row_swapped(r, half);
          const bool hide = mykey >= N || (CAUSAL && mykey > qidx);
          p = hide ? 0.f : p;
        }
        s[r] = p;
        dp[r] = p * (dp[r] - st_d[r]);
      }
      const bf16x8 p0 = pack_bf16(s, 0), p1 = pack_bf16(s, 8);
      const bf16x8 d0 = pack_bf16(dp, 0), d1 = pack_bf16(dp, 8);
      // dV += P^T dO and dK += dS^T Q (queries 32qb + 16t + 8*half + e)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const unsigned short* dot = smem + C::OFF_DOT + (32 * db + l32) * C::TS + 32 * qb + 8 * half;
        const unsigned short* qt = smem + C::OFF_QT + (32 * db + l32) * C::TS + 32 * qb + 8 * half;
        dv_acc[db] = mfma32(p0, lds_bf16x8(dot), dv_acc[db]);
        dv_acc[db] = mfma32(p1, lds_bf16x8(dot + 16), dv_acc[db]);
        dk_acc[db] = mfma32(d0, lds_bf16x8(qt), dk_acc[db]);
        dk_acc[db] = mfma32(d1, lds_bf16x8(qt + 16), dk_acc[db]);
      }
      // dS (bf16) to LDS, [query][key] with queries in natural order
      const uint4 u0 = as_uint4(d0), u1 = as_uint4(d1);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        ds_out[acc_row_swapped(r, half) * C::SS] = bf16_lane_of(u0, r);
        ds_out[acc_row_swapped(r + 8, half) * C::SS] = bf16_lane_of(u1, r);
      }
    }
    __syncthreads();  // dS complete; every wave is done with the Q / dO tile
    if (more) bwd_store_qtile<D>(smem, lse2, dlt, tid, regs);

    // dQ_tile (BM x D) += scale * dS (BM x 128 keys) K (128 keys x D): 32x32 blocks over the waves
    constexpr int NBLK = (BM / 32) * NDB;
    for (int blk = w; blk < NBLK; blk += 4) {
      const int qb = blk / NDB;
      const int db = blk % NDB;
      f32x16 acc = zero16();
      const unsigned short* arow = smem + C::OFF_DS + (32 * qb + l32) * C::SS + 8 * half;
      const unsigned short* brow = smem + C::OFF_KT + (32 * db + l32) * C::KTS + 8 * half;
#pragma unroll
      for (int kc = 0; kc < BN / 16; ++kc) acc = mfma32(lds_bf16x8(arow + 16 * kc), lds_bf16x8(brow + 16 * kc), acc);
      const int d = 32 * db + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qidx = q0 + 32 * qb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (qidx < N) unsafeAtomicAdd(a.dq_acc + hoff + (size_t)qidx * D + d, acc[r] * a.scale);
      }
    }
  }

  // ---- dK, dV out: C layout has lane = d column, registers = keys
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = 32 * db + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = wave_k0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key < N) {
        const size_t idx = hoff + (size_t)key * D + d;
        const float gk = dk_acc[db][r] * a.scale_abs;
        const float gv = dv_acc[db][r];
        if (a.grad_bf16) {
          static_cast<unsigned short*>(a.dk)[idx] = float_to_bf16_bits(gk);
          static_cast<unsigned short*>(a.dv)[idx] = float_to_bf16_bits(gv);
        } else {
          static_cast<float*>(a.dk)[idx] = gk;
          static_cast<float*>(a.dv)[idx] = gv;
        }
      }
    }
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
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  int BH;
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
  const int k0 = kt * BK;
  for (int idx = tid; idx < BK * D; idx += 64) {
    const int row = idx / D, col = idx % D;
    const int key = k0 + row;
    kk[row * (D + 1) + col] = key < N ? a.k[hoff + (size_t)key * D + col] : 0.f;
    vv[row * (D + 1) + col] = key < N ? a.v[hoff + (size_t)key * D + col] : 0.f;
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
      dl[tid] = row < N ? a.delta[hoff / D + row] : 0.f;
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
  const int tid = threadIdx.x;
  const int N = a.N;
  const int qt = (int)(blockIdx.x / a.BH);
  const int bh = (int)(blockIdx.x % a.BH);
  const size_t hoff = (size_t)bh * N * D;
  const int qi = qt * BQ + tid;
  const bool in = qi < N;
  float qv[D], dov[D], g[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qv[t] = in ? a.q[hoff + (size_t)qi * D + t] : 0.f;
    dov[t] = in ? a.dO[hoff + (size_t)qi * D + t] : 0.f;
    g[t] = 0.f;
  }
  const float l = in ? a.lse[hoff / D + qi] : -INFINITY;
  const float dl = in ? a.delta[hoff / D + qi] : 0.f;
  const int kend = CAUSAL ? min(N, qt * BQ + BQ) : N;
  for (int k0 = 0; k0 < kend; k0 += BK) {
    __syncthreads();
    for (int idx = tid; idx < BK * D; idx += 64) {
      const int row = k0 + idx / D;
      kk[idx] = row < N ? a.k[hoff + (size_t)row * D + idx % D] : 0.f;
      vv[idx] = row < N ? a.v[hoff + (size_t)row * D + idx % D] : 0.f;
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
// launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
static void launch_delta(const BwdParams& p, hipStream_t stream) {
  constexpr int EPT = 16 / sizeof(T);
  constexpr int RPB = 256 / (D / EPT);
  const long long rows = (long long)p.B * p.H * p.N;
  const unsigned blocks = (unsigned)((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3(blocks), dim3(256), 0, stream, static_cast<const T*>(p.o),
                     static_cast<const T*>(p.dO), p.delta, rows);
}

template <int D, bool CAUSAL>
static void launch_bwd_bf16_main(const BwdParams& p, hipStream_t stream) {
  BwdKernelArgs a;
  a.q = static_cast<const unsigned short*>(p.q);
  a.k = static_cast<const unsigned short*>(p.k);
  a.v = static_cast<const unsigned short*>(p.v);
  a.dO = static_cast<const unsigned short*>(p.dO);
  a.lse = p.lse;
  a.delta = p.delta;
  a.dq_acc = p.dq_acc;
  a.dk = p.dk;
  a.dv = p.dv;
  a.grad_bf16 = p.grad_dtype == 1;
  a.BH = p.B * p.H;
  a.N = p.N;
  const float sa = fabsf(p.scale);
  a.c = fmaxf(sa * kLog2e, 0x1p-100f);
  a.scale_abs = sa;
  a.scale = p.scale;
  a.neg = p.scale < 0.f ? 1 : 0;
  const int nkt = (p.N + 127) / 128;
  hipLaunchKernelGGL((bwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)(nkt * a.BH)), dim3(256), 0, stream, a);
}

template <int D, bool CAUSAL>
static void launch_bwd_f32(const BwdParams& p, hipStream_t stream) {
  BwdF32Args a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.dO = static_cast<const float*>(p.dO);
  a.lse = p.lse;
  a.delta = p.delta;
  a.dq = static_cast<float*>(p.dq);
  a.dk = static_cast<float*>(p.dk);
  a.dv = static_cast<float*>(p.dv);
  a.BH = p.B * p.H;
  a.N = p.N;
  a.scale = p.scale;
  const unsigned nk = (unsigned)((p.N + 63) / 64 * a.BH);
  hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, CAUSAL>), dim3(nk), dim3(64), 0, stream, a);
  hipLaunchKernelGGL((bwd_f32_dq_kernel<D, CAUSAL>), dim3(nk), dim3(64), 0, stream, a);
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  (void)hipGetLastError();  // clear an error left by an earlier, unrelated HIP call
  const long long rows = (long long)p.B * p.H * p.N;
  if (p.dtype == 0) {
    if (p.d == 64) {
      launch_delta<float, 64>(p, stream);
      if (p.causal) launch_bwd_f32<64, true>(p, stream); else launch_bwd_f32<64, false>(p, stream);
    } else {
      launch_delta<float, 128>(p, stream);
      if (p.causal) launch_bwd_f32<128, true>(p, stream); else launch_bwd_f32<128, false>(p, stream);
    }
    return hipGetLastError();
  }
  const long long n4 = rows * p.d / 4;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<float4*>(p.dq_acc), n4);
  if (p.d == 64) {
    launch_delta<unsigned short, 64>(p, stream);
    if (p.causal) launch_bwd_bf16_main<64, true>(p, stream); else launch_bwd_bf16_main<64, false>(p, stream);
  } else {
    launch_delta<unsigned short, 128>(p, stream);
    if (p.causal) launch_bwd_bf16_main<128, true>(p, stream); else launch_bwd_bf16_main<128, false>(p, stream);
  }
  if (p.grad_dtype == 1) {
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(p.dq_acc), static_cast<uint2*>(p.dq), n4);
  }
  return hipGetLastError();
}

}  // namespace fa
