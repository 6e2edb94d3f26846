/* A plain-C host program running one rank's share through libcpthd's C ABI on the GPU: its own device
 * buffers (hipMalloc / hipMemcpy), its own stream, no Python or torch.
 *
 *   consumer_gpu <in.bin> <out.bin>
 *
 * in.bin (little-endian): int32 T, cp, rank, strategy, num_docs, Hq, Hkv, D; float32 softmax scale;
 *   int32 cu_seqlens[num_docs + 1], cu_seqlens_padded[num_docs + 1];
 *   bf16 bits q_local[S*Hq*D], k[T*Hkv*D], v[T*Hkv*D], do_local[S*Hq*D]   (S = T / cp; K, V physical order)
 * out.bin: int32 idx[S] (partition indices); bf16 bits o[S*Hq*D]; float32 lse[S*Hq], dq[S*Hq*D],
 *   dk[T*Hkv*D], dv[T*Hkv*D].
 *
 * Steps: partition indices, the attention forward (which builds the plan in the workspace) and the
 * backward, into outputs first filled with NaN bits; every HIP and library status is checked, and the device
 * status word must stay 0.  Exit 0 on success.  Built by the build step beside this file; run and checked by tests/test_c_consumer.py. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cpthd.h"

#define HIP_OK(call)                                                                       \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) {                                                                \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));                   \
      return 2;                                                                            \
    }                                                                                      \
  } while (0)
#define LIB_OK(call)                                                                       \
  do {                                                                                     \
    int s_ = (call);                                                                       \
    if (s_ != CPTHD_OK) {                                                                  \
      fprintf(stderr, "%s returned %d: %s\n", #call, s_, cpthd_status_string(s_));         \
      return 3;                                                                            \
    }                                                                                      \
  } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) { return fread(dst, 1, bytes, f) == bytes ? 0 : 1; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
    return 1;
  }
  FILE* fin = fopen(argv[1], "rb");
  if (!fin) return 1;
  int32_t hdr[8];
  float scale;
  if (read_all(fin, hdr, sizeof hdr) || read_all(fin, &scale, sizeof scale)) return 1;
  const int32_t T = hdr[0], cp = hdr[1], rank = hdr[2], strategy = hdr[3], B = hdr[4], Hq = hdr[5], Hkv = hdr[6],
                D = hdr[7];
  if (T <= 0 || cp <= 0 || T % cp || B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return 1;
  const size_t S = (size_t)(T / cp), nq = S * Hq * D, nkv = (size_t)T * Hkv * D;
  int32_t* cu_a = malloc((B + 1) * sizeof(int32_t));
  int32_t* cu_p = malloc((B + 1) * sizeof(int32_t));
  uint16_t* q = malloc(nq * 2);
  uint16_t* k = malloc(nkv * 2);
  uint16_t* v = malloc(nkv * 2);
  uint16_t* dO = malloc(nq * 2);
  if (!cu_a || !cu_p || !q || !k || !v || !dO) return 1;
  if (read_all(fin, cu_a, (B + 1) * sizeof(int32_t)) || read_all(fin, cu_p, (B + 1) * sizeof(int32_t)) ||
      read_all(fin, q, nq * 2) || read_all(fin, k, nkv * 2) || read_all(fin, v, nkv * 2) || read_all(fin, dO, nq * 2))
    return 1;
  fclose(fin);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  const size_t ws_bytes = cpthd_attn_workspace_bytes(T, cp, Hq, Hkv, D, B);
  if (ws_bytes == 0) return 1;
  int32_t *d_cu_a, *d_cu_p, *d_idx, *d_status;
  void *d_q, *d_k, *d_v, *d_do, *d_o, *d_ws;
  float *d_lse, *d_dq, *d_dk, *d_dv;
  HIP_OK(hipMalloc((void**)&d_cu_a, (B + 1) * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&d_cu_p, (B + 1) * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&d_idx, S * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&d_status, sizeof(int32_t)));
  HIP_OK(hipMalloc(&d_q, nq * 2));
  HIP_OK(hipMalloc(&d_k, nkv * 2));
  HIP_OK(hipMalloc(&d_v, nkv * 2));
  HIP_OK(hipMalloc(&d_do, nq * 2));
  HIP_OK(hipMalloc(&d_o, nq * 2));
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMalloc((void**)&d_lse, S * Hq * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_dq, nq * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_dk, nkv * sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_dv, nkv * sizeof(float)));
  HIP_OK(hipMemcpy(d_cu_a, cu_a, (B + 1) * sizeof(int32_t), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_cu_p, cu_p, (B + 1) * sizeof(int32_t), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_q, q, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_k, k, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_v, v, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_do, dO, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(d_status, 0, sizeof(int32_t)));
  /* outputs start as NaN (all bits set): an entry the library leaves unwritten fails the comparison */
  HIP_OK(hipMemset(d_idx, 0xFF, S * sizeof(int32_t)));
  HIP_OK(hipMemset(d_o, 0xFF, nq * 2));
  HIP_OK(hipMemset(d_lse, 0xFF, S * Hq * sizeof(float)));
  HIP_OK(hipMemset(d_dq, 0xFF, nq * sizeof(float)));
  HIP_OK(hipMemset(d_dk, 0xFF, nkv * sizeof(float)));
  HIP_OK(hipMemset(d_dv, 0xFF, nkv * sizeof(float)));

  LIB_OK(cpthd_partition_indices(d_cu_p, B, T, cp, rank, strategy, d_idx, d_status, stream));
  LIB_OK(cpthd_attn_fwd(d_q, d_k, d_v, d_cu_a, d_cu_p, B, T, T, cp, rank, strategy, Hq, Hkv, D, scale, 1, -1, 0,
                        d_o, d_lse, d_ws, ws_bytes, d_status, stream));
  LIB_OK(cpthd_attn_bwd(d_q, d_k, d_v, d_o, d_do, d_lse, d_cu_a, d_cu_p, B, T, T, cp, rank, strategy, Hq, Hkv, D,
                        scale, 1, -1, 0, d_dq, d_dk, d_dv, d_ws, ws_bytes, d_status, stream));
  HIP_OK(hipStreamSynchronize(stream));
  int32_t status = -1;
  HIP_OK(hipMemcpy(&status, d_status, sizeof(int32_t), hipMemcpyDeviceToHost));
  if (status != 0) {
    fprintf(stderr, "device status %d\n", status);
    return 4;
  }

  int32_t* idx = malloc(S * sizeof(int32_t));
  uint16_t* o = malloc(nq * 2);
  float* lse = malloc(S * Hq * sizeof(float));
  float* dq = malloc(nq * sizeof(float));
  float* dk = malloc(nkv * sizeof(float));
  float* dv = malloc(nkv * sizeof(float));
  if (!idx || !o || !lse || !dq || !dk || !dv) return 1;
  HIP_OK(hipMemcpy(idx, d_idx, S * sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(o, d_o, nq * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, d_lse, S * Hq * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dq, d_dq, nq * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dk, d_dk, nkv * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dv, d_dv, nkv * sizeof(float), hipMemcpyDeviceToHost));
  FILE* fout = fopen(argv[2], "wb");
  if (!fout) return 1;
  fwrite(idx, sizeof(int32_t), S, fout);
  fwrite(o, 2, nq, fout);
  fwrite(lse, sizeof(float), S * Hq, fout);
  fwrite(dq, sizeof(float), nq, fout);
  fwrite(dk, sizeof(float), nkv, fout);
  fwrite(dv, sizeof(float), nkv, fout);
  fclose(fout);

  hipFree(d_cu_a); hipFree(d_cu_p); hipFree(d_idx); hipFree(d_status); hipFree(d_q); hipFree(d_k); hipFree(d_v);
  hipFree(d_do); hipFree(d_o); hipFree(d_ws); hipFree(d_lse); hipFree(d_dq); hipFree(d_dk); hipFree(d_dv);
  HIP_OK(hipStreamDestroy(stream));
  free(cu_a); free(cu_p); free(q); free(k); free(v); free(dO); free(idx); free(o); free(lse); free(dq); free(dk);
  free(dv);
  printf("ok\n");
  return 0;
}
