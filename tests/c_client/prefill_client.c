/*
 * A plain C client of the library's C ABI (include/sma.h): it reads one
 * prefill problem from binary files, runs sma_prefill (indexer -> top-k ->
 * sparse MLA) on the GPU through nothing but the HIP runtime's C API and
 * libsma.so, and writes the index lists, the output and the lse.  Test
 * infrastructure: tests/test_gpu_c_client.py compares what it writes with
 * the oracle and with the Python binding, so the boundary is exercised the
 * way a C or C++ caller would use it.
 *
 *   prefill_client DIR
 *
 * DIR/meta.txt   "n_q n_k h_idx d_idx top_k sm_scale"
 * DIR/q_idx.bin  bf16 bits [n_q, h_idx, d_idx]     DIR/w.bin     fp32 [n_q, h_idx]
 * DIR/k_idx.bin  bf16 bits [n_k, d_idx]            DIR/q.bin     bf16 bits [n_q, 64, 576]
 * DIR/kv.bin     bf16 bits [n_k, 576]              DIR/pos.bin   int32 [n_q]
 * writes DIR/idx.bin int32 [n_q, top_k], DIR/out.bin fp32 [n_q, 64, 512],
 * DIR/lse.bin fp32 [n_q, 64].  Exit status: 0 on success, 2 on a usage or
 * file error (before any GPU call), 1 on a HIP or library error.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sma.h"

static char g_dir[4096];

static const char* path_of(const char* name) {
  static char p[4200];
  snprintf(p, sizeof p, "%s/%s", g_dir, name);
  return p;
}

/* Reads exactly `bytes` bytes of DIR/name into a new host buffer. */
static void* read_file(const char* name, size_t bytes) {
  FILE* f = fopen(path_of(name), "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path_of(name));
    return NULL;
  }
  void* buf = malloc(bytes ? bytes : 1);
  const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
  const int extra = fgetc(f);
  fclose(f);
  if (!buf || got != bytes || extra != EOF) {
    fprintf(stderr, "%s: expected exactly %zu bytes\n", path_of(name), bytes);
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char* name, const void* buf, size_t bytes) {
  FILE* f = fopen(path_of(name), "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path_of(name));
    if (f) fclose(f);
    return 0;
  }
  return fclose(f) == 0;
}

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      goto done;                                                                  \
    }                                                                             \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2 || strlen(argv[1]) >= sizeof g_dir) {
    fprintf(stderr, "usage: %s DIR (see the header of prefill_client.c)\n", argv[0]);
    return 2;
  }
  strcpy(g_dir, argv[1]);
  int n_q = 0, h_idx = 0, d_idx = 0, top_k = 0;
  long long n_k = 0;
  float sm_scale = 0.f;
  FILE* mf = fopen(path_of("meta.txt"), "r");
  if (!mf || fscanf(mf, "%d %lld %d %d %d %f", &n_q, &n_k, &h_idx, &d_idx, &top_k, &sm_scale) != 6 || n_q < 1 ||
      n_k < 1 || h_idx < 1 || d_idx < 1 || top_k < 1) {
    fprintf(stderr, "bad or missing %s\n", path_of("meta.txt"));
    if (mf) fclose(mf);
    return 2;
  }
  fclose(mf);

  const size_t b_qi = (size_t)n_q * h_idx * d_idx * 2, b_w = (size_t)n_q * h_idx * 4;
  const size_t b_ki = (size_t)n_k * d_idx * 2, b_q = (size_t)n_q * SMA_HEADS * SMA_D_QK * 2;
  const size_t b_kv = (size_t)n_k * SMA_D_QK * 2, b_pos = (size_t)n_q * 4;
  const size_t b_idx = (size_t)n_q * top_k * 4, b_out = (size_t)n_q * SMA_HEADS * SMA_D_V * 4;
  const size_t b_lse = (size_t)n_q * SMA_HEADS * 4;
  void* h[6] = {read_file("q_idx.bin", b_qi), read_file("w.bin", b_w), read_file("k_idx.bin", b_ki),
                read_file("q.bin", b_q), read_file("kv.bin", b_kv), read_file("pos.bin", b_pos)};
  const size_t hb[6] = {b_qi, b_w, b_ki, b_q, b_kv, b_pos};
  int status = 2;
  void* d[6] = {0};
  void *d_idx_out = NULL, *d_out = NULL, *d_lse = NULL, *d_ws = NULL;
  void *h_idx_out = NULL, *h_out = NULL, *h_lse = NULL;
  for (int i = 0; i < 6; ++i)
    if (!h[i]) goto done;

  status = 1;
  for (int i = 0; i < 6; ++i) {
    HIP_OK(hipMalloc(&d[i], hb[i]));
    HIP_OK(hipMemcpy(d[i], h[i], hb[i], hipMemcpyHostToDevice));
  }
  const size_t ws_bytes = sma_workspace_bytes(SMA_OP_PREFILL, n_q, n_k, top_k, h_idx, d_idx);
  HIP_OK(hipMalloc(&d_idx_out, b_idx));
  HIP_OK(hipMalloc(&d_out, b_out));
  HIP_OK(hipMalloc(&d_lse, b_lse));
  HIP_OK(hipMalloc(&d_ws, ws_bytes ? ws_bytes : 1));

  const sma_status st = sma_prefill(d[0], d[1], h_idx, d[2], NULL, SMA_DT_BF16, d[3], d[4], NULL, SMA_DT_BF16,
                                    d[5], n_q, n_k, h_idx, d_idx, top_k, sm_scale, d_out, SMA_DT_FP32, d_lse,
                                    d_idx_out, d_ws, ws_bytes, NULL);
  if (st != SMA_OK) {
    fprintf(stderr, "sma_prefill returned %d: %s\n", (int)st, sma_last_error());
    goto done;
  }
  HIP_OK(hipDeviceSynchronize());
  h_idx_out = malloc(b_idx);
  h_out = malloc(b_out);
  h_lse = malloc(b_lse);
  if (!h_idx_out || !h_out || !h_lse) goto done;
  HIP_OK(hipMemcpy(h_idx_out, d_idx_out, b_idx, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_out, d_out, b_out, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_lse, d_lse, b_lse, hipMemcpyDeviceToHost));
  if (write_file("idx.bin", h_idx_out, b_idx) && write_file("out.bin", h_out, b_out) &&
      write_file("lse.bin", h_lse, b_lse)) {
    printf("prefill_client: n_q=%d n_k=%lld top_k=%d ok\n", n_q, n_k, top_k);
    status = 0;
  }

done:
  for (int i = 0; i < 6; ++i) {
    if (d[i]) hipFree(d[i]);
    free(h[i]);
  }
  if (d_idx_out) hipFree(d_idx_out);
  if (d_out) hipFree(d_out);
  if (d_lse) hipFree(d_lse);
  if (d_ws) hipFree(d_ws);
  free(h_idx_out);
  free(h_out);
  free(h_lse);
  return status;
}
