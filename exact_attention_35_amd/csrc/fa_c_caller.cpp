// fa_c_caller: a plain caller of the libfa.so C ABI, with no Python and no torch.
//
// It reads bf16 Q, K, V and dO from a file, runs fa_fwd and fa_bwd on the default
// stream with device buffers it allocates itself, and writes O (bf16), lse, dQ,
// dK and dV (fp32) to a second file; it also makes one call with an unsupported
// head dimension and prints the status string the library returns.  The tests
// use it to check the boundary as a C program sees it.
//
//   fa_c_caller <in> <out> B H N d causal
//   in : q, k, v, dO as little-endian bf16 bits, [B, H, N, d] each
//   out: o as bf16 bits [B, H, N, d], lse fp32 [B, H, N], dq, dk, dv fp32 [B, H, N, d]
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "fa.h"

static int fail(const char* what) {
  fprintf(stderr, "fa_c_caller: %s\n", what);
  return 1;
}

int main(int argc, char** argv) {
  if (argc != 8) return fail("usage: fa_c_caller <in> <out> B H N d causal");
  const int B = atoi(argv[3]), H = atoi(argv[4]), N = atoi(argv[5]), d = atoi(argv[6]), causal = atoi(argv[7]);
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return fail("bad shape");
  const size_t n = (size_t)B * H * N * d;  // elements of one [B, H, N, d] tensor
  const size_t rows = (size_t)B * H * N;

  unsigned short* host_in = (unsigned short*)malloc(4 * n * sizeof(unsigned short));
  if (!host_in) return fail("out of host memory");
  FILE* f = fopen(argv[1], "rb");
  if (!f) return fail("cannot open the input file");
  const size_t got = fread(host_in, sizeof(unsigned short), 4 * n, f);
  fclose(f);
  if (got != 4 * n) return fail("short input file");

  void *q, *k, *v, *dO, *o, *dq, *dk, *dv, *ws;
  float* lse;
  const size_t wsb = fa_bwd_workspace_size(B, H, N, d, FA_F32);
  if (hipMalloc(&q, 2 * n) != hipSuccess || hipMalloc(&k, 2 * n) != hipSuccess ||
      hipMalloc(&v, 2 * n) != hipSuccess || hipMalloc(&dO, 2 * n) != hipSuccess ||
      hipMalloc(&o, 2 * n) != hipSuccess || hipMalloc((void**)&lse, 4 * rows) != hipSuccess ||
      hipMalloc(&dq, 4 * n) != hipSuccess || hipMalloc(&dk, 4 * n) != hipSuccess ||
      hipMalloc(&dv, 4 * n) != hipSuccess || hipMalloc(&ws, wsb) != hipSuccess)
    return fail("hipMalloc failed");
  if (hipMemcpy(q, host_in, 2 * n, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(k, host_in + n, 2 * n, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(v, host_in + 2 * n, 2 * n, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dO, host_in + 3 * n, 2 * n, hipMemcpyHostToDevice) != hipSuccess)
    return fail("upload failed");

  const float scale = 1.0f / sqrtf((float)d);
  int st = fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, FA_BF16, NULL);
  if (st != FA_OK) return fail(fa_status_string(st));
  st = fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, FA_BF16, FA_F32, ws, wsb, NULL);
  if (st != FA_OK) return fail(fa_status_string(st));
  if (hipDeviceSynchronize() != hipSuccess) return fail("kernel execution failed");

  // an unsupported head dimension is rejected on the host, before any device work
  st = fa_fwd(q, k, v, o, lse, B, H, N, 96, scale, causal, FA_BF16, NULL);
  printf("d=96: %d %s\n", st, fa_status_string(st));

  unsigned short* host_o = (unsigned short*)malloc(2 * n);
  float* host_f = (float*)malloc(4 * (rows + 3 * n));
  if (!host_o || !host_f) return fail("out of host memory");
  if (hipMemcpy(host_o, o, 2 * n, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(host_f, lse, 4 * rows, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(host_f + rows, dq, 4 * n, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(host_f + rows + n, dk, 4 * n, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(host_f + rows + 2 * n, dv, 4 * n, hipMemcpyDeviceToHost) != hipSuccess)
    return fail("download failed");
  f = fopen(argv[2], "wb");
  if (!f) return fail("cannot open the output file");
  const int ok = fwrite(host_o, 2, n, f) == n && fwrite(host_f, 4, rows + 3 * n, f) == rows + 3 * n;
  fclose(f);
  if (!ok) return fail("short write");

  hipFree(q); hipFree(k); hipFree(v); hipFree(dO); hipFree(o); hipFree(lse);
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(ws);
  free(host_in); free(host_o); free(host_f);
  printf("fa_c_caller: ok (ABI version %d)\n", fa_version());
  return 0;
}
