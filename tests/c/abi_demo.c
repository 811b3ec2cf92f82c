/*
 * The block through its C ABI alone, from plain C: no Python, no torch.
 * Device memory comes from the HIP runtime's C API. A 300-token bf16 block
 * (d = 256, 2 heads x 128, F = 512) with seeded weights runs in place under
 * two chunk settings; the outputs must be bit-identical ("LayerStream: H3
 * Chunking": chunked output is bit-identical), finite and different from the
 * input, and the argument errors must come back as documented.
 * Exit status 0 and a final "abi_demo: ok" line mean success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dit_block.h"

#define CHECK_HIP(call)                                                       \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));       \
      return 1;                                                               \
    }                                                                         \
  } while (0)

static uint32_t lcg_state = 12345u;
static float urand(void) { /* uniform in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) * (2.0f / 16777216.0f) - 1.0f;
}
static uint16_t to_bf16(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* bf16 matrix of `n` values uniform in [-a, a), copied to the device */
static int dev_bf16(void** out, size_t n, float a) {
  uint16_t* h = (uint16_t*)malloc(n * sizeof(uint16_t));
  if (!h) return 1;
  for (size_t i = 0; i < n; ++i) h[i] = to_bf16(a * urand());
  CHECK_HIP(hipMalloc(out, n * sizeof(uint16_t)));
  CHECK_HIP(hipMemcpy(*out, h, n * sizeof(uint16_t), hipMemcpyHostToDevice));
  free(h);
  return 0;
}

static int run(dit_block* blk, const void* x0, void* x, const float* mod, int64_t n, int64_t d, int64_t ca,
               int64_t cm, uint16_t* host_out) {
  size_t ws_bytes = 0;
  int rc = dit_block_peak_workspace(blk, n, ca, cm, 0, &ws_bytes);
  if (rc != DIT_OK) {
    fprintf(stderr, "peak_workspace: %s\n", dit_block_strerror(rc));
    return 1;
  }
  void* ws = NULL;
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMemcpy(x, x0, (size_t)(n * d) * sizeof(uint16_t), hipMemcpyDeviceToDevice));
  rc = dit_block_forward(blk, x, mod, n, ca, cm, 0, ws, ws_bytes, NULL);
  if (rc != DIT_OK) {
    fprintf(stderr, "forward(%lld, %lld): %s\n", (long long)ca, (long long)cm, dit_block_strerror(rc));
    return 1;
  }
  /* too small a workspace is refused before anything is enqueued */
  if (dit_block_forward(blk, x, mod, n, ca, cm, 0, ws, ws_bytes - 256, NULL) != DIT_ENOSPC) {
    fprintf(stderr, "short workspace was not refused\n");
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(host_out, x, (size_t)(n * d) * sizeof(uint16_t), hipMemcpyDeviceToHost));
  CHECK_HIP(hipFree(ws));
  printf("abi_demo: forward (attn_chunk %lld, mlp_chunk %lld) with %zu workspace bytes\n", (long long)ca,
         (long long)cm, ws_bytes);
  return 0;
}

int main(void) {
  const int64_t d = 256, heads = 2, dh = 128, ffn = 512, n = 300;
  void *wqkv, *wo, *wgu, *wdown, *x0, *x;
  if (dev_bf16(&wqkv, (size_t)(3 * d * d), 0.1f) || dev_bf16(&wo, (size_t)(d * d), 0.1f) ||
      dev_bf16(&wgu, (size_t)(2 * ffn * d), 0.1f) || dev_bf16(&wdown, (size_t)(d * ffn), 0.07f) ||
      dev_bf16(&x0, (size_t)(n * d), 1.0f))
    return 1;
  CHECK_HIP(hipMalloc(&x, (size_t)(n * d) * sizeof(uint16_t)));
  float hmod[6 * 256];
  for (int i = 0; i < 6 * 256; ++i) hmod[i] = 0.3f * urand();
  float* mod = NULL;
  CHECK_HIP(hipMalloc((void**)&mod, sizeof(hmod)));
  CHECK_HIP(hipMemcpy(mod, hmod, sizeof(hmod), hipMemcpyHostToDevice));

  dit_block_desc desc = {d, heads, dh, ffn, DIT_BF16, 1e-6f};
  dit_block_weights w;
  memset(&w, 0, sizeof(w));
  w.w_qkv = wqkv;
  w.w_o = wo;
  w.w_gu = wgu;
  w.w_down = wdown;
  dit_block* blk = NULL;
  int rc = dit_block_create(&desc, &w, &blk);
  if (rc != DIT_OK) {
    fprintf(stderr, "create: %s\n", dit_block_strerror(rc));
    return 1;
  }
  /* argument errors are refused */
  dit_block_desc bad = desc;
  bad.head_dim = 96;
  dit_block* none = NULL;
  size_t bytes = 0;
  if (dit_block_create(&bad, &w, &none) != DIT_EINVAL || dit_block_peak_workspace(blk, n, 64, 0, 0, &bytes) != DIT_EINVAL) {
    fprintf(stderr, "invalid arguments were not refused\n");
    return 1;
  }

  uint16_t* y1 = (uint16_t*)malloc((size_t)(n * d) * sizeof(uint16_t));
  uint16_t* y2 = (uint16_t*)malloc((size_t)(n * d) * sizeof(uint16_t));
  uint16_t* xin = (uint16_t*)malloc((size_t)(n * d) * sizeof(uint16_t));
  if (!y1 || !y2 || !xin) return 1;
  CHECK_HIP(hipMemcpy(xin, x0, (size_t)(n * d) * sizeof(uint16_t), hipMemcpyDeviceToHost));
  if (run(blk, x0, x, mod, n, d, 0, n, y1) || run(blk, x0, x, mod, n, d, 64, 100, y2)) return 1;

  if (memcmp(y1, y2, (size_t)(n * d) * sizeof(uint16_t)) != 0) {
    fprintf(stderr, "outputs of the two chunk settings differ\n");
    return 1;
  }
  double sum = 0.0, moved = 0.0;
  for (int64_t i = 0; i < n * d; ++i) {
    const float v = from_bf16(y1[i]);
    if (!isfinite(v)) {
      fprintf(stderr, "non-finite output at %lld\n", (long long)i);
      return 1;
    }
    sum += v;
    moved += fabs((double)v - (double)from_bf16(xin[i]));
  }
  if (!(moved > 0.0)) {
    fprintf(stderr, "the block left x unchanged\n");
    return 1;
  }
  printf("abi_demo: outputs bit-identical across chunk settings; sum %.6f, mean |y - x| %.6f\n", sum,
         moved / (double)(n * d));
  dit_block_destroy(blk);
  free(y1);
  free(y2);
  free(xin);
  hipFree(wqkv);
  hipFree(wo);
  hipFree(wgu);
  hipFree(wdown);
  hipFree(x0);
  hipFree(x);
  hipFree(mod);
  printf("abi_demo: ok\n");
  return 0;
}
