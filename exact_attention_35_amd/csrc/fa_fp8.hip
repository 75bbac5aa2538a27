// FP8 (e4m3) path for gfx950: block quantisation with incoherent processing,
// and the FP8 attention forward.
//
// Method: the everydayai.blog flash-attention article, section
// "FlashAttention-3": FP8 arithmetic for speed, and incoherent processing to
// cut the quantisation error.  The pages define neither; the reading used:
//   * fp8 = OCP E4M3 (bias 7, largest finite 448, no infinities), the format of
//     the gfx950 matrix cores;
//   * one power-of-two scale per 128 consecutive rows of a head, the smallest
//     that maps the block's largest magnitude to at most 448;
//   * incoherent processing: Q and K rows are multiplied by diag(sigma) H_d (the
//     Sylvester Hadamard matrix, sigma random signs) before rounding; the
//     factor 1/sqrt(d) that makes the rotation orthogonal goes into the scale,
//     so (Q M)(K M)^T = Q K^T and the forward needs no change.
//
// quant_fp8_kernel: one workgroup per 128-row block, one row per lane.  The
// rotation is the fast Walsh-Hadamard transform in fp32, stages h = 1, 2, ...,
// d/2 in that order (the order fixes every rounding, so the codes are
// reproducible bit for bit); the block maximum sets the exponent; codes are
// rounded to nearest even by v_cvt_pk_fp8_f32.
//
// fwd_fp8_kernel: the bf16 forward's design (256 queries per workgroup, two
// groups of four waves in MFMA / softmax ping-pong, LDS-direct tile loads into
// rings of three buffers) on v_mfma_f32_32x32x64_f8f6f4:
//   * S^T = K Q^T: lane (query, half h) gets 16 keys of each 32-key block; K rows
//     sit in LDS permuted so that the two blocks of a 64-key group give lane h
//     exactly keys 32h .. 32h+31 in order, which are the k-slots of the P.V MFMA;
//   * P = exp2(S c_t - m) relative to a basis m that trails the running row
//     maximum by less than one binade (P <= 2, far inside e4m3's range; the
//     accumulator is rescaled only when the maximum passes m + 1), rounded to
//     e4m3 by v_cvt_pk_fp8_f32;
//   * O^T += V^T P^T, V^T read from the natural-order V tile by ds_read_b64_tr_b8
//     (each lane receives one d column of 8 keys per read);
//   * the per-block K scale enters the tile's score factor c_t = c qs ks_t; the
//     per-block V scale is applied by rescaling the accumulator when it changes
//     (the same branch as the rescale for a new row maximum).
#include <math.h>

#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// 32x32x64 fp8 x fp8 -> fp32 MFMA; operand format 0 (e4m3) on both sides and no
// block scales, which selects the unscaled instruction.  Operand layouts (gfx950):
//   A: lane l supplies row l % 32, k-slots 32 (l / 32) + byte 0 .. 31
//   B: lane l supplies column l % 32, k-slots 32 (l / 32) + byte 0 .. 31
//   C: as for the bf16 MFMA (register r of lane l: row 8(r/4) + 4(l/32) + r%4)
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// two fp32 values -> e4m3 bytes (round to nearest even) into the low or high half of `old`
template <bool HIGH>
__device__ __forceinline__ int cvt_fp8x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HIGH);
}

// ---------------------------------------------------------------------------
// quantisation
// ---------------------------------------------------------------------------
struct QuantArgs {
  const void* x;
  int x_f32;                 // 1: fp32 input, 0: bf16
  const signed char* signs;  // d random signs (negative = -1), or null: no rotation
  unsigned char* codes;
  float* scales;
  int N;
  int nb;       // 128-row blocks per head
  float rnorm;  // fl32(1 / sqrt(d)) when rotating, else 1
};

template <int D, bool F32>
__global__ __launch_bounds__(128) void quant_fp8_kernel(QuantArgs a) {
  // The block's rows move between HBM and LDS in coalesced 16-byte pieces (thread t
  // takes pieces t, t + 128, ...); each lane then works on one row in registers.
  // Rows are padded by 16 bytes in LDS so that the 64 lanes' row reads spread over
  // the banks.
  constexpr int XROW = D * (F32 ? 4 : 2) + 16;  // LDS bytes per input row
  constexpr int CROW = D + 16;              // LDS bytes per code row
  __shared__ __align__(16) unsigned char xs[128 * XROW];
  __shared__ float wmax[2];
  const int tid = (int)threadIdx.x;
  const int blk = (int)blockIdx.x;  // bh * nb + block
  const int bh = blk / a.nb;
  const int r0 = (blk - bh * a.nb) * 128;
  const int rows = min(128, a.N - r0);
  const int row = r0 + tid;
  const bool in = tid < rows;
  constexpr int rbytes = D * (F32 ? 4 : 2);
  {
    // every load of the thread is issued before the first LDS store, so that all of
    // them are in flight together
    constexpr int PT = rbytes / 16;  // 16-byte pieces per thread (= per row)
    const unsigned char* src = static_cast<const unsigned char*>(a.x) + ((size_t)bh * a.N + r0) * rbytes;
    const int pieces = rows * PT;
    uint4 v[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = tid + 128 * j;
      v[j] = i < pieces ? *reinterpret_cast<const uint4*>(src + 16 * (size_t)i) : zero_uint4();
    }
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = tid + 128 * j;
      *reinterpret_cast<uint4*>(xs + (i / PT) * XROW + 16 * (i % PT)) = v[j];
    }
  }
  __syncthreads();
  float y[D];
  if (F32) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const float4 f = in ? *reinterpret_cast<const float4*>(xs + tid * XROW + 16 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
      y[4 * i] = f.x;
      y[4 * i + 1] = f.y;
      y[4 * i + 2] = f.z;
      y[4 * i + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const uint4 u = in ? *reinterpret_cast<const uint4*>(xs + tid * XROW + 16 * i) : zero_uint4();
#pragma unroll
      for (int e = 0; e < 8; ++e) y[8 * i + e] = bf16_bits_to_float(bf16_lane_of(u, e));
    }
  }
  if (a.signs != nullptr) {
#pragma unroll
    for (int i = 0; i < D; ++i) y[i] = a.signs[i] < 0 ? -y[i] : y[i];
    // y <- y H_d, stage by stage; each butterfly rounds its sum and difference once
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        if ((i & h) == 0) {
          const float u = y[i], w = y[i + h];
          y[i] = u + w;
          y[i + h] = u - w;
        }
      }
    }
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) m = fmaxf(m, fabsf(y[i]));
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();  // also: every lane has read its row, so xs can take the codes
  const float amax = fmaxf(wmax[0], wmax[1]);
  // smallest e with amax 2^-e <= 448 = 0.875 2^9 (exact: frexp splits amax into mantissa and exponent)
  int e = 0;
  if (amax > 0.f) {
    int ex;
    const float mant = frexpf(amax, &ex);
    e = mant <= 0.875f ? ex - 9 : ex - 8;
  }
  if (tid == 0) a.scales[blk] = ldexpf(a.rnorm, e);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    unsigned int w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* p = y + 16 * i + 4 * j;
      int v = cvt_fp8x2<false>(ldexpf(p[0], -e), ldexpf(p[1], -e), 0);
      v = cvt_fp8x2<true>(ldexpf(p[2], -e), ldexpf(p[3], -e), v);
      w[j] = (unsigned int)v;
    }
    *reinterpret_cast<uint4*>(xs + tid * CROW + 16 * i) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  __syncthreads();
  {
    constexpr int PT = D / 16;
    unsigned char* dst = a.codes + ((size_t)bh * a.N + r0) * D;
    const int pieces = rows * PT;
    uint4 v[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = tid + 128 * j;
      v[j] = *reinterpret_cast<const uint4*>(xs + (i / PT) * CROW + 16 * (i % PT));
    }
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int i = tid + 128 * j;
      if (i < pieces) *reinterpret_cast<uint4*>(dst + 16 * (size_t)i) = v[j];
    }
  }
  (void)row;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
struct Fp8FwdArgs {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  const float* qs;  // [B, H, nb] scales of Q's 128-row blocks
  const float* ks;  // [B, H_kv, nb]
  const float* vs;  // [B, H_kv, nb]
  unsigned short* o;
  float* lse;
  int BH;
  int group;  // query heads per K/V head
  int N;
  int nb;
  float c;  // |scale| * log2(e), clamped away from 0
  int neg;  // scale < 0: Q's sign bits are flipped on load
};

// 16-byte chunk swizzle of an fp8 tile row: the 8 rows read together by a
// 128-byte LDS cycle (8 consecutive rows of a 16-byte column for the K operand
// reads, 8 consecutive keys of a 16-byte column for the transposing V reads)
// land on distinct banks.  d = 128: rows are one bank line; d = 64: two rows
// share a line, so the swizzle uses the row bits above the lowest.
template <int D>
__device__ __forceinline__ int swz8(int row) {
  return D == 128 ? (row & 7) : ((row >> 1) & 3);
}

// Key stored at LDS row p of a 64-key group of the K tile.  S^T register r of
// lane half h in 32-row block b reads row 32b + 8(r/4) + 4h + r%4; storing key
// 32h + 16b + r there makes byte 16b + r of lane h's P fragment key 32h + 16b + r.
__device__ __forceinline__ int perm8(int p) {
  return (((p >> 2) & 1) << 5) | (((p >> 5) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}

template <int D, int BN>
struct Fp8Cfg {
  static constexpr int TILE = BN * D;                 // bytes of a K or V tile
  static constexpr int LPW = TILE / 1024 / 4;          // 1 KB loads per wave (4 waves per tile)
  static constexpr int NSB = BN / 32;                 // 32-key S^T blocks
  static constexpr int NPG = BN / 64;                 // 64-key P fragments
  static constexpr int NDB = D / 32;                  // 32-wide d blocks of O
  static constexpr int NDC = D / 64;                  // 64-wide d chunks of S^T = K Q^T
  static constexpr int BM = 256;
  static_assert(LPW * 4 * 1024 == TILE, "a tile is a whole number of 1 KB loads per wave");
  static constexpr int NH = BN > 128 ? BN / 128 : 1;  // 128-row K/V scale blocks per tile
  static_assert(128 % BN == 0 || BN % 128 == 0, "a key tile covers whole scale blocks or lies inside one");
};

template <int D, int BN>
__device__ __forceinline__ void dma_k8(BufRes res, unsigned char* buf, int kt, int wi, int lane) {
  using C = Fp8Cfg<D, BN>;
#pragma unroll
  for (int n = 0; n < C::LPW; ++n) {
    const int blk = wi * C::LPW + n;
    const int p = blk * (1024 / D) + lane / (D / 16);  // LDS row written by this lane
    const int c = (lane % (D / 16)) ^ swz8<D>(p);      // 16-byte chunk that belongs there
    const int key = (p & ~63) | perm8(p & 63);
    const unsigned int off = (unsigned int)((kt * BN + key) * D + 16 * c);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void_t*)(buf + blk * 1024), 16, off, 0, 0, 0);
  }
}

template <int D, int BN>
__device__ __forceinline__ void dma_v8(BufRes res, unsigned char* buf, int kt, int wi, int lane) {
  using C = Fp8Cfg<D, BN>;
#pragma unroll
  for (int n = 0; n < C::LPW; ++n) {
    const int blk = wi * C::LPW + n;
    const int p = blk * (1024 / D) + lane / (D / 16);
    const int c = (lane % (D / 16)) ^ swz8<D>(p);
    const unsigned int off = (unsigned int)((kt * BN + p) * D + 16 * c);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void_t*)(buf + blk * 1024), 16, off, 0, 0, 0);
  }
}

__device__ __forceinline__ uint4 lds_u4(const unsigned char* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ i32x8 join8(uint4 lo, uint4 hi) {
  i32x8 r;
  r[0] = (int)lo.x;
  r[1] = (int)lo.y;
  r[2] = (int)lo.z;
  r[3] = (int)lo.w;
  r[4] = (int)hi.x;
  r[5] = (int)hi.y;
  r[6] = (int)hi.z;
  r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ i32x2 lds_tr8(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)((__attribute__((address_space(3))) unsigned char*)p));
}

// S^T = K Q^T for one tile: block b (keys 64(b/2) + 32h + 16(b%2) + r for register r
// of lane half h), accumulated over the 64-wide d chunks.
template <int D, int BN>
__device__ __forceinline__ void qk_tile8(const unsigned char* kbuf, const int (&ko)[2 * (D / 64)],
                                         const i32x8 (&qf)[D / 64], f32x16 (&s)[BN / 32]) {
  int o[2 * (D / 64)];
#pragma unroll
  for (int i = 0; i < 2 * (D / 64); ++i) o[i] = fresh(ko[i]);
#pragma unroll
  for (int b = 0; b < BN / 32; ++b) s[b] = zero16();
#pragma unroll
  for (int cc = 0; cc < D / 64; ++cc) {
#pragma unroll
    for (int b = 0; b < BN / 32; ++b) {
      const unsigned char* base = kbuf + 32 * b * D;
      s[b] = mfma_fp8(join8(lds_u4(base + o[2 * cc]), lds_u4(base + o[2 * cc + 1])), qf[cc], s[b]);
    }
  }
}

// O^T += V^T P^T: d block db, 64-key group g; the V^T operand (keys 64g + 32h + j for
// byte j, d = 32 db + lane % 32) comes from four transposing reads of 8 keys each.
// A 256-key tile spans two V scale blocks: the accumulator, expressed in the first
// block's scale, is multiplied by `mid` (first / second scale) before the second
// half is added (a uniform branch, taken only when the two scales differ).
template <int D, int BN>
__device__ __forceinline__ void pv_tile8(const unsigned char* vbuf, const int (&vo)[D / 32],
                                         const i32x8 (&pf)[BN / 64], f32x16 (&oacc)[D / 32], float mid) {
  int o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = fresh(vo[db]);
#pragma unroll
  for (int g = 0; g < BN / 64; ++g) {
    if (BN > 128 && g == 2 && mid != 1.f) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= mid;
      }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned char* p = vbuf + 64 * g * D + o[db];
      i32x8 a;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x2 t = lds_tr8(p + 8 * q * D);
        a[2 * q] = t[0];
        a[2 * q + 1] = t[1];
      }
      oacc[db] = mfma_fp8(a, pf[g], oacc[db]);
    }
  }
}

// keys past N, and under causal masking keys after the query, get -inf
template <int BN, bool CAUSAL>
__device__ __forceinline__ void mask_tile8(f32x16 (&s)[BN / 32], int k_first, int qrow, int N, int half) {
#pragma unroll
  for (int b = 0; b < BN / 32; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k_first + 64 * (b >> 1) + 32 * half + 16 * (b & 1) + r;
      const bool hide = key >= N || (CAUSAL && key > qrow);
      s[b][r] = hide ? -INFINITY : s[b][r];
    }
  }
}

// this lane's maximum of S ct over the tile (ct per 128-key scale block), across both half-waves
template <int BN, int NH>
__device__ __forceinline__ float tile_max8(const f32x16 (&s)[BN / 32], const float (&ct)[NH]) {
  constexpr int NB = BN / 32 / NH;  // 32-key blocks per scale block
  float mt = -INFINITY;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int b0 = h * NB;
    float m = max3f(s[b0][0], s[b0][1], s[b0][2]);
#pragma unroll
    for (int i = 3; i + 1 < 16 * NB; i += 2)
      m = max3f(m, s[b0 + (i >> 4)][i & 15], s[b0 + ((i + 1) >> 4)][(i + 1) & 15]);
    m = max2f(m, s[b0 + NB - 1][15]);
    mt = NH == 1 ? m * ct[0] : max2f(mt, m * ct[h]);
  }
  return xhalf_max(mt);
}

// P = exp2(S ct - mc) -> e4m3 fragments (byte 16b' + r of fragment g from block 2g + b');
// returns the fp32 sum of this half-wave's P
template <int BN, int NH>
__device__ __forceinline__ float exp_tile8(const f32x16 (&s)[BN / 32], const float (&cts)[NH], float mc,
                                           i32x8 (&pf)[BN / 64]) {
  float lsum = 0.f;
#pragma unroll
  for (int g = 0; g < BN / 64; ++g) {
    const float ct = cts[(2 * g) / (BN / 32 / NH)];  // the scale block of this 64-key group
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int b = 2 * g + (w >> 2);
      const int r = 4 * (w & 3);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[b][r], ct, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[b][r + 1], ct, -mc));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(s[b][r + 2], ct, -mc));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(s[b][r + 3], ct, -mc));
      lsum += (p0 + p1) + (p2 + p3);
      // both halves are overwritten: passing the previous tile's (consumed) fragment as
      // the preserved input lets the conversion write in place, without zeroing first
      pf[g][w] = cvt_fp8x2<true>(p2, p3, cvt_fp8x2<false>(p0, p1, pf[g][w]));
    }
  }
  return lsum;
}

template <int D, int BN>
__device__ __forceinline__ void sched_gemm_phase8() {
  constexpr int NPV = (BN / 64) * (D / 32);
  constexpr int NQK = (BN / 32) * (D / 64);
#pragma unroll
  for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  }
#pragma unroll
  for (int i = 0; i < NQK; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(512) void fwd_fp8_kernel(Fp8FwdArgs a) {
  using C = Fp8Cfg<D, BN>;
  constexpr int BM = C::BM;
  constexpr int NSB = C::NSB;
  constexpr int NPG = C::NPG;
  constexpr int NDB = C::NDB;
  constexpr int NDC = C::NDC;
  __shared__ __align__(16) unsigned char kbuf_0[C::TILE];
  __shared__ __align__(16) unsigned char kbuf_1[C::TILE];
  __shared__ __align__(16) unsigned char kbuf_2[C::TILE];
  __shared__ __align__(16) unsigned char vbuf_0[C::TILE];
  __shared__ __align__(16) unsigned char vbuf_1[C::TILE];
  __shared__ __align__(16) unsigned char vbuf_2[C::TILE];

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
  const GridPos gp = grid_pos<HR>(nqt, a.BH);
  const int qt = CAUSAL ? nqt - 1 - gp.r : gp.r;  // longest rows first
  const int bh = gp.bh;
  const int kvh = bh / a.group;
  const unsigned int head_bytes = (unsigned int)N * D;
  const BufRes qres = make_buf(a.q + (size_t)bh * N * D, head_bytes);
  const BufRes kres = make_buf(a.k + (size_t)kvh * N * D, head_bytes);
  const BufRes vres = make_buf(a.v + (size_t)kvh * N * D, head_bytes);
  const BufRes ores = make_buf(a.o + (size_t)bh * N * D, head_bytes * 2);
  const float* ks = a.ks + (size_t)kvh * a.nb;
  const float* vs = a.vs + (size_t)kvh * a.nb;

  const int q_first = qt * BM;
  const int wave_q0 = q_first + 32 * (2 * wg + grp);
  const int qrow = wave_q0 + l32;
  const int kend = CAUSAL ? min(N, q_first + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  auto tile_at = [&](int t) __attribute__((always_inline)) -> int { return min(t, ntiles - 1); };
  auto need_mask = [&](int kt) __attribute__((always_inline)) -> bool {
    const int k_first = kt * BN;
    return (k_first + BN > N) || (CAUSAL && k_first + BN - 1 > wave_q0);
  };

  // this lane's query row as MFMA B fragments (d = 64 cc + 32 half .. +31)
  i32x8 qf[NDC];
  {
    const unsigned int sign = a.neg ? 0x80808080u : 0u;
#pragma unroll
    for (int cc = 0; cc < NDC; ++cc) {
      uint4 lo = buf_load16(qres, (unsigned int)(qrow * D + 64 * cc + 32 * half));
      uint4 hi = buf_load16(qres, (unsigned int)(qrow * D + 64 * cc + 32 * half + 16));
      lo.x ^= sign; lo.y ^= sign; lo.z ^= sign; lo.w ^= sign;
      hi.x ^= sign; hi.y ^= sign; hi.z ^= sign; hi.w ^= sign;
      qf[cc] = join8(lo, hi);
    }
  }
  const float qscale = a.qs[(size_t)bh * a.nb + min(wave_q0 / 128, a.nb - 1)];
  const float cq = a.c * qscale;
  // K operand reads: LDS row l32 of each 32-row block, chunks 4cc + 2h and 4cc + 2h + 1
  int ko[2 * NDC];
#pragma unroll
  for (int cc = 0; cc < NDC; ++cc) {
#pragma unroll
    for (int j = 0; j < 2; ++j) ko[2 * cc + j] = l32 * D + (((4 * cc + 2 * half + j) ^ swz8<D>(l32)) * 16);
  }
  // V^T operand reads: 16-lane group G = lane / 16 covers keys 32 (G / 2) + 8q + (lane % 16) / 2 and
  // d columns 32 db + 16 (G % 2) + 8 (lane % 2) .. +7 per lane
  int vo[NDB];
  {
    const int G = lane >> 4;
    const int c = lane & 15;
    const int row = 32 * (G >> 1) + (c >> 1);
#pragma unroll
    for (int db = 0; db < NDB; ++db) vo[db] = row * D + (((2 * db + (G & 1)) ^ swz8<D>(row)) * 16) + 8 * (c & 1);
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  float m2 = -INFINITY;  // running row maximum of S c_t (log2 units)
  float l_half = 0.f;
  float vbase = 1.f;  // V scale the accumulator is expressed in
  float pv_mid = 1.f;   // for the pending P.V of a two-block tile: first / second V scale,
  float pv_vlast = 1.f; // and the second one
  f32x16 s[NSB];
  i32x8 pf[NPG];
#pragma unroll
  for (int b = 0; b < NSB; ++b) s[b] = zero16();
#pragma unroll
  for (int g = 0; g < NPG; ++g) pf[g] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};

  // V buffers start as zeros: the first MFMA phase multiplies buffer 2 by P = 0
  for (int i = tid; i < C::TILE / 16; i += 512) {
    reinterpret_cast<uint4*>(vbuf_0)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_1)[i] = zero_uint4();
    reinterpret_cast<uint4*>(vbuf_2)[i] = zero_uint4();
  }
  barrier_lds();
  if (grp == 1) {
    dma_k8<D, BN>(kres, kbuf_0, tile_at(0), wg, lane);
    dma_k8<D, BN>(kres, kbuf_1, tile_at(1), wg, lane);
  } else {
    dma_v8<D, BN>(vres, vbuf_0, tile_at(0), wg, lane);
    wait_dma();
  }
  barrier_ring<C::LPW>();

  auto gemm_phase = [&](int t, const unsigned char* kcur, const unsigned char* vprev) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    pv_tile8<D, BN>(vprev, vo, pf, oacc, pv_mid);
    if (C::NH > 1) vbase = pv_vlast;  // the accumulator is now in the second block's scale
    qk_tile8<D, BN>(kcur, ko, qf, s);
    sched_gemm_phase8<D, BN>();
    if (t < ntiles) {
      const int kt = tile_at(t);
      if (need_mask(kt)) mask_tile8<BN, CAUSAL>(s, kt * BN, qrow, N, half);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto softmax_phase = [&](int t) __attribute__((always_inline)) {
    constexpr int NH = C::NH;
    const int blk = (tile_at(t) * BN) >> 7;
    float ct[NH];
    float vh[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int bi = min(blk + h, a.nb - 1);  // a second block wholly past N only holds masked keys
      ct[h] = fmaxf(cq * ks[bi], 0x1p-100f);
      vh[h] = vs[bi];
    }
    const float vt = vh[0];
    if (NH > 1) {
      pv_mid = vh[0] / vh[NH - 1];
      pv_vlast = vh[NH - 1];
    }
    const float mt = tile_max8<BN, NH>(s, ct);
    // the basis moves only when the maximum exceeds it by more than one binade, so P <= 2
    // (far inside e4m3's range) and most tiles skip the accumulator rescale
    const bool grow = mt > m2 + 1.f;
    float alpha = 1.f;
    if (grow) {
      alpha = __builtin_amdgcn_exp2f(m2 - mt);
      m2 = mt;
    }
    if (__ballot(grow) || vt != vbase) {
      const float f = alpha * (vbase / vt);
#pragma unroll
      for (int i = 0; i < NDB; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= f;
      }
      vbase = vt;
    }
    const float mc = m2 == -INFINITY ? 0.f : m2;
    l_half = l_half * alpha + exp_tile8<BN, NH>(s, ct, mc, pf);
  };
  auto step = [&](int t, const unsigned char* kcur, unsigned char* knext2, const unsigned char* vprev,
                  unsigned char* vnext) __attribute__((always_inline)) {
    if (grp == 0) {
      dma_v8<D, BN>(vres, vnext, tile_at(t + 1), wg, lane);
      gemm_phase(t, kcur, vprev);
    } else {
      if (t >= 1) softmax_phase(t - 1);
    }
    barrier_plain();
    if (grp == 0) {
      if (t < ntiles) softmax_phase(t);
    } else {
      dma_k8<D, BN>(kres, knext2, tile_at(t + 2), wg, lane);
      gemm_phase(t, kcur, vprev);
    }
    barrier_ring<C::LPW>();
  };
  for (int t = 0; t <= ntiles; t += 3) {
    step(t, kbuf_0, kbuf_2, vbuf_2, vbuf_1);
    if (t + 1 <= ntiles) step(t + 1, kbuf_1, kbuf_0, vbuf_0, vbuf_2);
    if (t + 2 <= ntiles) step(t + 2, kbuf_2, kbuf_1, vbuf_1, vbuf_0);
  }
  wait_dma();

  // ---- epilogue: O = acc vbase / l (bf16), lse = m ln 2 + ln l
  const float l = xhalf_sum(l_half);
  const float inv = l > 0.f ? vbase / l : 0.f;
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
      buf_store8(ores, (unsigned int)(qrow * D + d0) * 2, pk);
    }
  }
  if (a.lse != nullptr && half == 0 && qrow < N) {
    a.lse[(size_t)bh * N + qrow] = l > 0.f ? m2 * 0.6931471805599453f + logf(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_fp8_quantize(const Fp8QuantParams& p, hipStream_t stream) {
  (void)hipGetLastError();
  QuantArgs a;
  a.x = p.x;
  a.x_f32 = p.dtype == 0 ? 1 : 0;
  a.signs = p.signs;
  a.codes = p.codes;
  a.scales = p.scales;
  a.N = p.N;
  a.nb = (p.N + 127) / 128;
  a.rnorm = p.signs != nullptr ? (float)(1.0 / sqrt((double)p.d)) : 1.0f;
  const dim3 grid((unsigned)((size_t)p.B * p.H * a.nb));
  if (p.d == 64) {
    if (a.x_f32) hipLaunchKernelGGL((quant_fp8_kernel<64, true>), grid, dim3(128), 0, stream, a);
    else hipLaunchKernelGGL((quant_fp8_kernel<64, false>), grid, dim3(128), 0, stream, a);
  } else {
    if (a.x_f32) hipLaunchKernelGGL((quant_fp8_kernel<128, true>), grid, dim3(128), 0, stream, a);
    else hipLaunchKernelGGL((quant_fp8_kernel<128, false>), grid, dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D, int BN, bool CAUSAL>
static hipError_t launch_fp8_fwd_t(const Fp8FwdParams& p, hipStream_t stream) {
  Fp8FwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.qs = p.qs;
  a.ks = p.ks;
  a.vs = p.vs;
  a.o = static_cast<unsigned short*>(p.o);
  a.lse = p.lse;
  a.BH = p.B * p.H;
  a.group = p.H / p.Hkv;
  a.N = p.N;
  a.nb = (p.N + 127) / 128;
  a.c = fmaxf(fabsf(p.scale) * kLog2e, 0x1p-100f);
  a.neg = p.scale < 0.f ? 1 : 0;
  const int nqt = (p.N + 255) / 256;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, BN, CAUSAL>), dim3((unsigned)(nqt * a.BH)), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fp8_fwd(const Fp8FwdParams& p, hipStream_t stream) {
  (void)hipGetLastError();
  // 16 KB tiles: 128 keys (one K/V scale block) at d = 128, 256 keys (two) at d = 64 -- except
  // for short sequences, where the half-empty last tile of 256 keys costs more than it saves
  if (p.d == 64 && p.N <= 2048)
    return p.causal ? launch_fp8_fwd_t<64, 128, true>(p, stream) : launch_fp8_fwd_t<64, 128, false>(p, stream);
  if (p.d == 64)
    return p.causal ? launch_fp8_fwd_t<64, 256, true>(p, stream) : launch_fp8_fwd_t<64, 256, false>(p, stream);
  return p.causal ? launch_fp8_fwd_t<128, 128, true>(p, stream) : launch_fp8_fwd_t<128, 128, false>(p, stream);
}

}  // namespace fa
