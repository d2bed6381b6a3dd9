/* A plain C11 caller of the library's C ABI: no Python, no torch.
 *
 * usage: forward_from_c DIR T E TOP_K K N
 *
 * Reads the inputs of one contiguous-layout problem (fp8 UE8M0 activations,
 * 128x128 block-scaled fp8 weights, SiLU(gate) * up) as raw little-endian
 * arrays from DIR, allocates device memory with hipMalloc, runs moe_forward
 * on the default stream and writes DIR/out.bin:
 *   hidden.bin      bf16  [T, K]
 *   topk_ids.bin    int32 [T, TOP_K]
 *   topk_w.bin      fp32  [T, TOP_K]
 *   is_padding.bin  uint8 [T]            (optional)
 *   w13.bin         e4m3  [E, 2N, K]     w13_sf.bin fp32 [E, 2N/128, K/128]
 *   w2.bin          e4m3  [E, K, N]      w2_sf.bin  fp32 [E, K/128, N/128]
 *   out.bin         bf16  [T, K]         (written)
 * Exit status 0 on success; a library error prints moe_last_error().
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_fp8.h"

static void* read_file(const char* dir, const char* name, size_t bytes, int optional) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (f == NULL) {
    if (optional) return NULL;
    fprintf(stderr, "cannot open %s\n", path);
    exit(2);
  }
  void* buf = malloc(bytes > 0 ? bytes : 1);
  if (buf == NULL || fread(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path);
    exit(2);
  }
  fclose(f);
  return buf;
}

static void* to_device(const void* host, size_t bytes) {
  void* dev = NULL;
  if (hipMalloc(&dev, bytes > 0 ? bytes : 1) != hipSuccess ||
      hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "device copy of %zu bytes failed\n", bytes);
    exit(3);
  }
  return dev;
}

int main(int argc, char** argv) {
  if (argc != 7) {
    fprintf(stderr, "usage: %s DIR T E TOP_K K N\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  const int T = atoi(argv[2]), E = atoi(argv[3]), k = atoi(argv[4]);
  const int K = atoi(argv[5]), N = atoi(argv[6]);

  moe_problem_t p;
  memset(&p, 0, sizeof p);
  p.num_tokens = T;
  p.hidden = K;
  p.intermediate = N;
  p.num_experts = E;
  p.top_k = k;
  p.layout = MOE_LAYOUT_CONTIGUOUS;
  p.act_quant = MOE_Q_FP8_UE8M0;
  p.weight_quant = MOE_W_FP8_BLOCK128;
  p.activation = MOE_ACT_SILU;

  const size_t n_hidden = (size_t)T * K * 2, n_slots = (size_t)T * k;
  const size_t n_w13 = (size_t)E * 2 * N * K, n_w13_sf = (size_t)E * (2 * N / 128) * (K / 128) * 4;
  const size_t n_w2 = (size_t)E * K * N, n_w2_sf = (size_t)E * (K / 128) * (N / 128) * 4;
  void* h_hidden = read_file(dir, "hidden.bin", n_hidden, 0);
  void* h_ids = read_file(dir, "topk_ids.bin", n_slots * 4, 0);
  void* h_w = read_file(dir, "topk_w.bin", n_slots * 4, 0);
  void* h_pad = read_file(dir, "is_padding.bin", (size_t)T, 1);
  void* h_w13 = read_file(dir, "w13.bin", n_w13, 0);
  void* h_w13_sf = read_file(dir, "w13_sf.bin", n_w13_sf, 0);
  void* h_w2 = read_file(dir, "w2.bin", n_w2, 0);
  void* h_w2_sf = read_file(dir, "w2_sf.bin", n_w2_sf, 0);

  size_t ws_bytes = 0;
  if (moe_workspace_size(&p, &ws_bytes) != MOE_OK) {
    fprintf(stderr, "moe_workspace_size: %s\n", moe_last_error());
    return 4;
  }
  void* d_hidden = to_device(h_hidden, n_hidden);
  void* d_ids = to_device(h_ids, n_slots * 4);
  void* d_w = to_device(h_w, n_slots * 4);
  void* d_pad = h_pad != NULL ? to_device(h_pad, (size_t)T) : NULL;
  void* d_w13 = to_device(h_w13, n_w13);
  void* d_w13_sf = to_device(h_w13_sf, n_w13_sf);
  void* d_w2 = to_device(h_w2, n_w2);
  void* d_w2_sf = to_device(h_w2_sf, n_w2_sf);
  void *d_out = NULL, *d_ws = NULL;
  if (hipMalloc(&d_out, n_hidden > 0 ? n_hidden : 1) != hipSuccess ||
      hipMalloc(&d_ws, ws_bytes > 0 ? ws_bytes : 1) != hipSuccess) {
    fprintf(stderr, "hipMalloc failed\n");
    return 3;
  }

  const moe_status_t st = moe_forward(&p, d_hidden, NULL, (const int32_t*)d_ids,
                                      (const float*)d_w, (const uint8_t*)d_pad, NULL, d_w13,
                                      d_w13_sf, d_w2, d_w2_sf, d_out, d_ws, ws_bytes, NULL);
  if (st != MOE_OK) {
    fprintf(stderr, "moe_forward: %s\n", moe_last_error());
    return 4;
  }
  if (hipDeviceSynchronize() != hipSuccess) {
    fprintf(stderr, "hipDeviceSynchronize failed\n");
    return 3;
  }
  void* h_out = malloc(n_hidden > 0 ? n_hidden : 1);
  if (h_out == NULL || hipMemcpy(h_out, d_out, n_hidden, hipMemcpyDeviceToHost) != hipSuccess) {
    fprintf(stderr, "copy back failed\n");
    return 3;
  }
  char path[4096];
  snprintf(path, sizeof path, "%s/out.bin", dir);
  FILE* f = fopen(path, "wb");
  if (f == NULL || fwrite(h_out, 1, n_hidden, f) != n_hidden) {
    fprintf(stderr, "cannot write %s\n", path);
    return 2;
  }
  fclose(f);
  printf("forward_from_c: T=%d E=%d top_k=%d K=%d N=%d workspace %zu bytes: ok\n", T, E, k, K, N,
         ws_bytes);
  hipFree(d_hidden); hipFree(d_ids); hipFree(d_w); hipFree(d_pad); hipFree(d_w13);
  hipFree(d_w13_sf); hipFree(d_w2); hipFree(d_w2_sf); hipFree(d_out); hipFree(d_ws);
  free(h_hidden); free(h_ids); free(h_w); free(h_pad); free(h_w13); free(h_w13_sf);
  free(h_w2); free(h_w2_sf); free(h_out);
  return 0;
}
