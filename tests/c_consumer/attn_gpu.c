/* The attention path driven from plain C: HIP runtime API and
 * include/calibatt.h only, no Python or torch in the process.
 *
 *   attn_gpu IN OUT
 *
 * IN holds int32 H, int32 N, float scale, then bf16 bits of q, k and v
 * ([H][N][128] each, contiguous) and the uint8 block mask [H][R][R]
 * (R = ceil(N / 128)). The program uploads them, compiles the mask into
 * kept-block lists on the device (calibatt_compile_skiplist), runs
 * calibatt_sparse_attn_fwd on the default stream and writes the bf16 bits
 * of o to OUT; it also runs calibatt_sparse_attn_fwd_noalloc (no workspace)
 * and reports whether its output is byte-identical. Exit status 0 on
 * success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "calibatt.h"

#define HIP_OK(call)                                                         \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
      return 2;                                                              \
    }                                                                        \
  } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) {
  return fread(dst, 1, bytes, f) == bytes ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: attn_gpu IN OUT\n");
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 1;
  int32_t H = 0, N = 0;
  float scale = 0.f;
  if (read_all(in, &H, 4) || read_all(in, &N, 4) || read_all(in, &scale, 4) || H <= 0 || N <= 0)
    return 1;
  const int32_t R = (N + 127) / 128;
  const size_t tbytes = (size_t)H * N * 128 * 2, mbytes = (size_t)H * R * R;
  uint16_t* host = (uint16_t*)malloc(3 * tbytes);
  uint8_t* mask = (uint8_t*)malloc(mbytes);
  if (!host || !mask || read_all(in, host, 3 * tbytes) || read_all(in, mask, mbytes)) return 1;
  fclose(in);

  void *q, *k, *v, *o, *o2, *ws;
  uint8_t* d_mask;
  int32_t *off, *idx;
  const size_t ws_bytes = calibatt_sparse_attn_fwd_workspace(H, N);
  HIP_OK(hipMalloc(&q, tbytes));
  HIP_OK(hipMalloc(&k, tbytes));
  HIP_OK(hipMalloc(&v, tbytes));
  HIP_OK(hipMalloc(&o, tbytes));
  HIP_OK(hipMalloc(&o2, tbytes));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMalloc((void**)&d_mask, mbytes));
  HIP_OK(hipMalloc((void**)&off, ((size_t)H * R + 1) * 4));
  HIP_OK(hipMalloc((void**)&idx, mbytes * 4));
  HIP_OK(hipMemcpy(q, host, tbytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, (const char*)host + tbytes, tbytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, (const char*)host + 2 * tbytes, tbytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_mask, mask, mbytes, hipMemcpyHostToDevice));

  int64_t nnz = 0;
  int rc = calibatt_compile_skiplist(d_mask, H, R, off, idx, &nnz, NULL);
  if (rc != CALIBATT_OK) {
    fprintf(stderr, "calibatt_compile_skiplist: %d %s\n", rc, calibatt_last_error());
    return 3;
  }
  rc = calibatt_sparse_attn_fwd(q, k, v, o, H, N, 128, (int64_t)N * 128, 128, scale, off, idx, nnz,
                                NULL, NULL, ws, ws_bytes, NULL);
  if (rc != CALIBATT_OK) {
    fprintf(stderr, "calibatt_sparse_attn_fwd: %d %s\n", rc, calibatt_last_error());
    return 3;
  }
  rc = calibatt_sparse_attn_fwd_noalloc(q, k, v, o2, H, N, 128, (int64_t)N * 128, 128, scale, off, idx,
                                        nnz, NULL, NULL, NULL);
  if (rc != CALIBATT_OK) {
    fprintf(stderr, "calibatt_sparse_attn_fwd_noalloc: %d %s\n", rc, calibatt_last_error());
    return 3;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(host, o, tbytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy((char*)host + tbytes, o2, tbytes, hipMemcpyDeviceToHost));
  const int same = memcmp(host, (const char*)host + tbytes, tbytes) == 0;
  FILE* out = fopen(argv[2], "wb");
  if (!out || fwrite(host, 1, tbytes, out) != tbytes) return 1;
  fclose(out);
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(o);
  hipFree(o2);
  hipFree(ws);
  hipFree(d_mask);
  hipFree(off);
  hipFree(idx);
  free(host);
  free(mask);
  printf("ok nnz=%lld noalloc=%s\n", (long long)nnz, same ? "equal" : "different");
  return 0;
}
