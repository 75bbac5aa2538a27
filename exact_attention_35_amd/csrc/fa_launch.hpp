// Host-side launchers of the attention kernels (internal to libfa.so).
// Arguments have been validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  void* o_lo;                 // bf16 only: low-order part of O, bf16(O - bf16(O)); may be null
  float* lse;                 // may be null
  const unsigned char* mask;  // block-sparse tile mask, null when dense
  int B, H, N, d;
  int Hkv;  // K/V heads (divides H); query head h reads K/V head h / (H / Hkv)
  float scale;
  int causal;
  int dtype;  // FA_F32 / FA_BF16
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* o_lo;  // bf16 only: low-order part of O (D is then formed from o + o_lo); may be null
  const float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  float* stats;  // workspace: per row of [B, H, N], the pair (lse * log2 e, -D) with D = rowsum(dO * O)
  // workspace, grouped-query only (Hkv < H): fp32 dK and dV of every query head, [B, H, N, d] each,
  // summed over each group into dk / dv by a final kernel
  float* part_k;
  float* part_v;
  const unsigned char* mask;  // block-sparse tile mask (bf16 only), null when dense
  int B, H, N, d;
  int Hkv;
  float scale;
  int causal;
  int dtype;
  int grad_dtype;
};

// FP8 path (e4m3 codes, per-128-row block scales)
struct Fp8QuantParams {
  const void* x;
  int dtype;                 // FA_F32 / FA_BF16
  const signed char* signs;  // null: no rotation
  unsigned char* codes;
  float* scales;
  int B, H, N, d;
};

struct Fp8FwdParams {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  const float* qs;
  const float* ks;
  const float* vs;
  void* o;     // bf16
  float* lse;  // may be null
  int B, H, Hkv, N, d;
  float scale;
  int causal;
};

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
hipError_t launch_fp8_quantize(const Fp8QuantParams& p, hipStream_t stream);
hipError_t launch_fp8_fwd(const Fp8FwdParams& p, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

}  // namespace fa
