// C ABI of libfa.so: argument validation (no HIP call before it passes), then
// dispatch to the kernel launchers.  Semantics and error codes are documented
// in include/fa.h.
#include "fa.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa_launch.hpp"

namespace {

constexpr long long kMaxGrid = 0x7fffffffLL;
constexpr size_t kLdsBytes = 160 * 1024;  // gfx950 LDS per workgroup
// static LDS of the bf16 forward: K and V tiles of 16 KB, three buffers each, plus at most
// 256 bytes of bookkeeping (list lengths, the row-pairing counts)
constexpr size_t kFwdStaticLds = (size_t)6 * 16384 + 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_common(int B, int H, int N, int d, float scale, int causal, int dtype) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (d < 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // every grid is at most B*H*ceil(N/64) workgroups and element offsets are 64-bit
  const long long bh = (long long)B * (long long)H;
  if (bh > kMaxGrid) return FA_ERR_INVALID_ARG;
  if (bh * (((long long)N + 63) / 64) > kMaxGrid) return FA_ERR_INVALID_ARG;
  // one head's [N, d] slice is addressed with 32-bit byte offsets
  if ((long long)N * d * 4 > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

size_t elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// grouped-query: H_kv K/V heads, each shared by H / H_kv consecutive query heads
bool valid_kv_heads(int H, int Hkv) { return Hkv >= 1 && Hkv <= H && H % Hkv == 0; }

int fwd_impl(const void* q, const void* k, const void* v, const unsigned char* mask, void* o, void* o_lo,
             float* lse, int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype, void* stream,
             bool sparse) {
  int st = check_common(B, H, N, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (!valid_kv_heads(H, Hkv)) return FA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (sparse && !mask) return FA_ERR_INVALID_ARG;
  if (o_lo && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)) ||
      (o_lo && !aligned16(o_lo)))
    return FA_ERR_INVALID_ARG;
  const size_t n = (size_t)B * H * N;
  const size_t tb = n * d * elem_bytes(dtype);
  const size_t kvb = (size_t)B * Hkv * N * d * elem_bytes(dtype);
  const Range in[3] = {range_of(q, tb), range_of(k, kvb), range_of(v, kvb)};
  // outputs: o, then the optional lse and o_lo (an empty range when absent)
  const Range outs[3] = {range_of(o, tb), range_of(lse, lse ? n * 4 : 0), range_of(o_lo, o_lo ? tb : 0)};
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : in)
      if (overlap(outs[i], r)) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
  }
  if (sparse) {
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    const size_t nb = ((size_t)N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
    // the kernel lists the kept mask columns of its two mask rows (uint16 each) in dynamic LDS
    const size_t list_bytes = (2 * nb * 2 + 15) & ~(size_t)15;
    if (kFwdStaticLds + list_bytes > kLdsBytes) return FA_ERR_UNSUPPORTED;
    const Range rm = range_of(mask, nb * nb);
    for (const Range& r : outs)
      if (overlap(rm, r)) return FA_ERR_INVALID_ARG;
  }
  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.o_lo = o_lo;
  p.lse = lse;
  p.mask = sparse ? mask : nullptr;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal;
  p.dtype = dtype;
  const hipError_t e = fa::launch_fwd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK:
      return "FA_OK: success";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG: invalid argument (null or misaligned pointer, bad size, enum or scale, or "
             "an output overlapping an input)";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: unsupported configuration (head dim must be 64 or 128; block-sparse is bf16 "
             "only; bf16 gradients need bf16 inputs)";
    case FA_ERR_WORKSPACE:
      return "FA_ERR_WORKSPACE: workspace missing or smaller than fa_bwd_workspace_size()";
    case FA_ERR_HIP:
      return "FA_ERR_HIP: a HIP kernel launch failed";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: fa_bwd_noalloc needs more workspace than its static device buffer holds "
             "(FA_NOALLOC_SCRATCH_BYTES = 32 MiB); use fa_bwd_ex with a caller workspace";
    default:
      return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* stream) {
  return fwd_impl(q, k, v, nullptr, o, nullptr, lse, B, H, H, N, d, scale, causal, dtype, stream, false);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
               int d, float scale, int causal, int dtype, void* stream) {
  return fwd_impl(q, k, v, nullptr, o, nullptr, lse, B, H, H_kv, N, d, scale, causal, dtype, stream, false);
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, const unsigned char* block_mask, void* o,
                       float* lse, int B, int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  return fwd_impl(q, k, v, block_mask, o, nullptr, lse, B, H, H, N, d, scale, causal, dtype, stream, true);
}

int fa_fwd_blocksparse_gqa(const void* q, const void* k, const void* v, const unsigned char* block_mask, void* o,
                           float* lse, int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype,
                           void* stream) {
  return fwd_impl(q, k, v, block_mask, o, nullptr, lse, B, H, H_kv, N, d, scale, causal, dtype, stream, true);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, const unsigned char* block_mask, void* o, void* o_lo,
              float* lse, int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype, void* stream) {
  return fwd_impl(q, k, v, block_mask, o, o_lo, lse, B, H, H_kv, N, d, scale, causal, dtype, stream,
                  block_mask != nullptr);
}

size_t fa_bwd_gqa_workspace_size(int B, int H, int H_kv, int N, int d, int grad_dtype) {
  if (check_common(B, H, N, d, 1.0f, 0, grad_dtype) != FA_OK || !valid_kv_heads(H, H_kv)) return 0;
  const size_t n = (size_t)B * H * N;
  size_t bytes = n * 8;  // per row: (lse * log2 e, D), two fp32
  if (H_kv < H) bytes = ((bytes + 255) & ~(size_t)255) + 2 * n * d * 4;  // fp32 dK, dV per query head
  return bytes;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d, int grad_dtype) {
  return fa_bwd_gqa_workspace_size(B, H, H, N, d, grad_dtype);
}

}  // extern "C"

namespace {

// static LDS of the block-sparse backward kernels (tile rings, hand-over buffers, bookkeeping)
constexpr size_t bwd_dkdv_static_lds(int d) { return d == 128 ? 132608 + 64 : 83456 + 64; }
constexpr size_t kBwdDqStaticLds = (size_t)6 * 16384 + 256;

// ---- the static workspace of fa_bwd_noalloc: one array per GPU, alive until the process ends.
// In host code `scratch` only names the variable; its device address on the current GPU comes
// from hipGetSymbolAddress, taken once per device and kept.
constexpr size_t kScratchBytes = (size_t)FA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current GPU's scratch array, or null on a HIP error.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// use_scratch: the workspace is the static scratch array (workspace and workspace_bytes are
// ignored); checked against its size, and its address taken only after every other check.
int bwd_impl(const void* q, const void* k, const void* v, const unsigned char* mask, const void* o, const void* o_lo,
             const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
             float scale, int causal, int dtype, int grad_dtype, void* workspace, size_t workspace_bytes,
             void* stream, bool sparse, bool use_scratch = false) {
  int st = check_common(B, H, N, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (!valid_kv_heads(H, Hkv)) return FA_ERR_INVALID_ARG;
  if (grad_dtype != FA_F32 && grad_dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (dtype == FA_F32 && grad_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (o_lo && (dtype != FA_BF16 || !aligned16(o_lo))) return FA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  if (sparse) {
    if (!mask) return FA_ERR_INVALID_ARG;
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    // the kernels list the kept rows of a mask column / columns of two mask rows in LDS
    const size_t nb = ((size_t)N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
    if (bwd_dkdv_static_lds(d) + ((nb * 2 + 15) & ~(size_t)15) > kLdsBytes) return FA_ERR_UNSUPPORTED;
    if (kBwdDqStaticLds + ((nb * 4 + 15) & ~(size_t)15) > kLdsBytes) return FA_ERR_UNSUPPORTED;
  }
  const size_t need = fa_bwd_gqa_workspace_size(B, H, Hkv, N, d, grad_dtype);
  if (use_scratch) {
    if (need > kScratchBytes) return FA_ERR_SCRATCH;
    workspace = nullptr;  // its range (below) is empty: the static array is no caller buffer
  } else {
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_INVALID_ARG;
  }
  const size_t n = (size_t)B * H * N;
  const size_t nkv = (size_t)B * Hkv * N;
  const size_t tb = n * d * elem_bytes(dtype);
  const size_t kvb = nkv * d * elem_bytes(dtype);
  const size_t gb = n * d * elem_bytes(grad_dtype);
  const size_t gkvb = nkv * d * elem_bytes(grad_dtype);
  const Range ins[7] = {range_of(q, tb),      range_of(k, kvb), range_of(v, kvb),
                        range_of(o, tb),      range_of(lse, n * 4), range_of(dO, tb),
                        range_of(o_lo, o_lo ? tb : 0)};
  const Range outs[4] = {range_of(dq, gb), range_of(dk, gkvb), range_of(dv, gkvb),
                         range_of(workspace, workspace ? need : 0)};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
    if (sparse) {
      const size_t nb = ((size_t)N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
      if (overlap(outs[i], range_of(mask, nb * nb))) return FA_ERR_INVALID_ARG;
    }
  }
  if (use_scratch) {
    workspace = scratch_on_current_device();
    if (workspace == nullptr) return FA_ERR_HIP;
  }
  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.o_lo = o_lo;
  p.lse = lse;
  p.dO = dO;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.stats = static_cast<float*>(workspace);
  p.part_k = nullptr;
  p.part_v = nullptr;
  if (Hkv < H) {
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((n * 8 + 255) & ~(size_t)255));
    p.part_k = part;
    p.part_v = part + n * d;
  }
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal;
  p.dtype = dtype;
  p.grad_dtype = grad_dtype;
  p.mask = sparse ? mask : nullptr;
  const hipError_t e = fa::launch_bwd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
           void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype, int grad_dtype,
           void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, nullptr, o, nullptr, lse, dO, dq, dk, dv, B, H, H, N, d, scale, causal,
                  dtype, grad_dtype, workspace, workspace_bytes, stream, false);
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
               void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal, int dtype,
               int grad_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, nullptr, o, nullptr, lse, dO, dq, dk, dv, B, H, H_kv, N, d, scale, causal,
                  dtype, grad_dtype, workspace, workspace_bytes, stream, false);
}

int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const unsigned char* block_mask, const void* o,
                       const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                       float scale, int causal, int dtype, int grad_dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return bwd_impl(q, k, v, block_mask, o, nullptr, lse, dO, dq, dk, dv, B, H, H, N, d, scale, causal,
                  dtype, grad_dtype, workspace, workspace_bytes, stream, true);
}

int fa_bwd_blocksparse_gqa(const void* q, const void* k, const void* v, const unsigned char* block_mask,
                           const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                           int H, int H_kv, int N, int d, float scale, int causal, int dtype, int grad_dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, block_mask, o, nullptr, lse, dO, dq, dk, dv, B, H, H_kv, N, d, scale, causal,
                  dtype, grad_dtype, workspace, workspace_bytes, stream, true);
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const unsigned char* block_mask, const void* o,
              const void* o_lo, const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
              int H_kv, int N, int d, float scale, int causal, int dtype, int grad_dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, block_mask, o, o_lo, lse, dO, dq, dk, dv, B, H, H_kv, N, d, scale, causal, dtype,
                  grad_dtype, workspace, workspace_bytes, stream, block_mask != nullptr);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const unsigned char* block_mask, const void* o,
                   const void* o_lo, const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                   int H_kv, int N, int d, float scale, int causal, int dtype, int grad_dtype, void* stream) {
  return bwd_impl(q, k, v, block_mask, o, o_lo, lse, dO, dq, dk, dv, B, H, H_kv, N, d, scale, causal, dtype,
                  grad_dtype, nullptr, 0, stream, block_mask != nullptr, /*use_scratch=*/true);
}

}  // extern "C"

namespace {

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" {

int fa_quantize_fp8(const void* x, const signed char* signs, unsigned char* codes, float* scales, int B, int H,
                    int N, int d, int dtype, void* stream) {
  int st = check_common(B, H, N, d, 1.0f, 0, dtype);
  if (st != FA_OK) return st;
  if (!x || !codes || !scales) return FA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned4(scales)) return FA_ERR_INVALID_ARG;
  const size_t n = (size_t)B * H * N;
  const size_t nb = ((size_t)N + FA_FP8_BLOCK - 1) / FA_FP8_BLOCK;
  if ((size_t)B * H * nb > (size_t)kMaxGrid) return FA_ERR_INVALID_ARG;
  const Range rx = range_of(x, n * d * elem_bytes(dtype));
  const Range rc = range_of(codes, n * d);
  const Range rs = range_of(scales, (size_t)B * H * nb * 4);
  if (overlap(rx, rc) || overlap(rx, rs) || overlap(rc, rs)) return FA_ERR_INVALID_ARG;
  if (signs) {
    const Range rg = range_of(signs, (size_t)d);
    if (overlap(rg, rc) || overlap(rg, rs)) return FA_ERR_INVALID_ARG;
  }
  fa::Fp8QuantParams p;
  p.x = x;
  p.dtype = dtype;
  p.signs = signs;
  p.codes = codes;
  p.scales = scales;
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  const hipError_t e = fa::launch_fp8_quantize(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const unsigned char* q, const unsigned char* k, const unsigned char* v, const float* q_scale,
               const float* k_scale, const float* v_scale, void* o, float* lse, int B, int H, int H_kv, int N, int d,
               float scale, int causal, void* stream) {
  int st = check_common(B, H, N, d, scale, causal, FA_BF16);
  if (st != FA_OK) return st;
  if (!valid_kv_heads(H, H_kv)) return FA_ERR_INVALID_ARG;
  if (!q || !k || !v || !q_scale || !k_scale || !v_scale || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_INVALID_ARG;
  if (!aligned4(q_scale) || !aligned4(k_scale) || !aligned4(v_scale)) return FA_ERR_INVALID_ARG;
  const size_t n = (size_t)B * H * N;
  const size_t nkv = (size_t)B * H_kv * N;
  const size_t nb = ((size_t)N + FA_FP8_BLOCK - 1) / FA_FP8_BLOCK;
  const Range ins[6] = {range_of(q, n * d), range_of(k, nkv * d), range_of(v, nkv * d),
                        range_of(q_scale, (size_t)B * H * nb * 4), range_of(k_scale, (size_t)B * H_kv * nb * 4),
                        range_of(v_scale, (size_t)B * H_kv * nb * 4)};
  const Range ro = range_of(o, n * d * 2);
  for (const Range& r : ins) {
    if (overlap(ro, r)) return FA_ERR_INVALID_ARG;
    if (lse && overlap(range_of(lse, n * 4), r)) return FA_ERR_INVALID_ARG;
  }
  if (lse && overlap(range_of(lse, n * 4), ro)) return FA_ERR_INVALID_ARG;
  fa::Fp8FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.qs = q_scale;
  p.ks = k_scale;
  p.vs = v_scale;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Hkv = H_kv;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.causal = causal;
  const hipError_t e = fa::launch_fp8_fwd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
