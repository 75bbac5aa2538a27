// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA operand layouts used throughout (CDNA4, wave64, v_mfma_f32_32x32x16_bf16):
//   A (32 x 16): lane l supplies row (l % 32), k-slots 8*(l/32) .. 8*(l/32)+7
//   B (16 x 32): lane l supplies column (l % 32), k-slots 8*(l/32) .. +7
//   C (32 x 32): lane l holds column (l % 32); accumulator register r holds
//                row 8*(r/4) + 4*(l/32) + (r%4)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_uint4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ bf16x8 lds_bf16x8(const unsigned short* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Eight fp32 values -> bf16x8, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16(const f32x16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[base + e];
  return r;
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short b) {
  return __uint_as_float(((unsigned int)b) << 16);
}

__device__ __forceinline__ unsigned short float_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(unsigned short, h);
}

// Swap bits 2 and 3 of a row index inside its 32-row group.  Rows of an MFMA
// A-operand tile are stored in LDS in this order so that the accumulator
// registers 0..7 / 8..15 of lane l hold 8 *consecutive* keys (or queries),
// 16*(r/8) + 8*(l/32) + (r%8), which is what the next MFMA's k-slots need.
__device__ __forceinline__ int swap23(int row) {
  return (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);
}

// Key (or query) offset within a 32-row block held by accumulator register r of
// an MFMA whose A rows were stored with swap23.
__device__ __forceinline__ int acc_row_swapped(int r, int half) {
  return 16 * (r >> 3) + 8 * half + (r & 7);
}

// max of three fp32 values in one v_max3_f32 (fmaxf would first canonicalize
// every input, doubling the instruction count; the scores are never NaN)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

__device__ __forceinline__ float max2f(float a, float b) {
  float d;
  asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Combine a value across the two half-waves (lanes l and l ^ 32) with
// v_permlane32_swap: each lane ends up holding {own, partner} in the pair.
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Bits of element e (0..7) of eight packed bf16 values.
__device__ __forceinline__ unsigned short bf16_lane_of(const uint4& u, int e) {
  const unsigned int w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
  return (unsigned short)((e & 1) ? (w >> 16) : (w & 0xffffu));
}

__device__ __forceinline__ uint4 zero_uint4() { return make_uint4(0u, 0u, 0u, 0u); }

// Consecutive workgroups of a launch go to the chip's eight XCDs in turn, and each
// XCD has an L2 of its own.  xcd_run(i, G) renumbers workgroup i of G (a bijection on
// [0, G)) so that the workgroups one XCD receives, in launch order, carry consecutive
// numbers.
__device__ __forceinline__ int xcd_run(int i, int G) {
  constexpr int NX = 8;
  const int per = (G + NX - 1) / NX;             // workgroups of the fuller XCDs
  const int full = G % NX == 0 ? NX : G % NX;    // how many XCDs receive `per`
  const int x = i % NX;
  const int j = i / NX;
  return x < full ? x * per + j : full * per + (x - full) * (per - 1) + j;
}

// Position of this workgroup in a grid of nrow * BH workgroups: its rank r in the
// head's launch order and its head bh.  Either way each XCD serves B*H/8 heads when
// B*H is a multiple of 8.  By default consecutive workgroups take consecutive heads
// at one rank, so every XCD runs all ranks of a causal grid longest first.  With
// HEAD_RUNS, B*H a multiple of 8 and more workgroups than the chip holds at once
// (more than four per CU), each XCD works through its heads one after the other, so
// the workgroups it runs at one time read the same head's tiles through its L2.  That
// pays where rows are of like length or short against the whole launch (grids without
// causal masking, block-sparse rows), and costs a tail in a dense causal grid, where
// each head's longest rows would start late.
struct GridPos {
  int r;
  int bh;
};
// Causal grids (rows longest first): each XCD takes its heads g at a time, rank-major
// inside a group, with g the smallest power of two, at least 2, for which a group's
// work (about g nrow^2 / 2 row steps over `slots` resident workgroups) outlasts its
// longest row (nrow steps): the XCD's resident workgroups then read the K/V of g heads
// through its L2 instead of those of all its heads, without starting any long row late.
// When it would leave a single group (or B*H is not a multiple of 8) the order is the
// default one of grid_pos.
__device__ __forceinline__ GridPos grid_pos_causal(int nrow, int BH, int slots) {
  const int i = (int)blockIdx.x;
  const int hx = BH >> 3;  // heads per XCD
  int g = 2;
  while (g < hx && g * nrow < 2 * slots) g <<= 1;
  if ((BH & 7) != 0 || g >= hx || hx % g != 0) return {i / BH, i % BH};
  const int G = (int)gridDim.x;
  const int L = xcd_run(i, G);
  const int per = G >> 3;
  const int x = L / per;
  const int j = L - x * per;
  const int grp = j / (g * nrow);
  const int rem = j - grp * g * nrow;
  return {rem / g, x * hx + grp * g + rem % g};
}

template <bool HEAD_RUNS>
__device__ __forceinline__ GridPos grid_pos(int nrow, int BH) {
  const int i = (int)blockIdx.x;
  const int G = (int)gridDim.x;
  if (HEAD_RUNS && (BH & 7) == 0 && G > 1024) {
    const int L = xcd_run(i, G);
    return {L % nrow, L / nrow};
  }
  return {i / BH, i % BH};
}

// ---- buffer (V#) memory access: the hardware range check returns zeros for
// loads past `bytes` and drops stores past it, so tails need no branches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t BufRes;

__device__ __forceinline__ BufRes make_buf(const void* base, unsigned int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(BufRes r, unsigned int byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void buf_store8(BufRes r, unsigned int byte_off, uint2 x) {
  u32x2 v;
  v[0] = x.x;
  v[1] = x.y;
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 0);
}

}  // namespace fa
