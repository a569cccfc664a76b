/* A torch-free caller of the C ABI on the GPU: three delayed-scaling steps of
 * a small FC1-shaped layer (X [M x K] and W [K x N], bf16, both E4M3), each
 * followed by the FP8 GEMM C = X_q * W_q with fp32 output, driven only
 * through include/fp8mi.h and the HIP runtime's C API.
 *
 * Usage: fc1_from_c OUTDIR.  The program generates its inputs (a fixed linear
 * congruential sequence, rounded to bf16), runs the steps and writes, per
 * step t, the inputs and everything the library produced as raw files in
 * OUTDIR, so that the calling test can replay the steps with the CPU oracle:
 *   x<t>.bin  bf16 [M x K]     w<t>.bin  bf16 [K x N]
 *   qx<t>.bin uint8 [M x K]    qwt<t>.bin uint8 [N x K]   c<t>.bin fp32 [M x N]
 *   sx<t>.bin, sw<t>.bin: fp32 {amax, scale, scale_inv, scale_inv_used},
 *                         then int32 {head, status}, then fp32 history[16]
 * Prints one line per step; exits non-zero on the first failed call. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8mi.h"

enum { M = 256, K = 512, N = 384, L = 16, STEPS = 3 };

static uint32_t g_state = 12345u;

/* Roughly normal values in [-2, 2): a sum of four uniforms. */
static float draw(void) {
  float s = 0.0f;
  for (int i = 0; i < 4; ++i) {
    g_state = g_state * 1664525u + 1013904223u;
    s += (float)(g_state >> 8) * (1.0f / 16777216.0f);
  }
  return s - 2.0f;
}

/* bf16 bit pattern of a finite float, rounded to nearest even. */
static uint16_t to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

#define HIP_OK(call)                                                            \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
      exit(2);                                                                  \
    }                                                                           \
  } while (0)

#define FP8_OK(call)                                                            \
  do {                                                                          \
    int s_ = (call);                                                            \
    if (s_ != FP8MI_OK) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, fp8mi_status_string(s_));       \
      exit(3);                                                                  \
    }                                                                           \
  } while (0)

static void write_file(const char* dir, const char* name, int t, const void* p, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s%d.bin", dir, name, t);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, n, f) != n) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(4);
  }
  fclose(f);
}

/* One tensor's delayed-scaling state on the device. */
typedef struct {
  float *history, *amax, *scale, *scale_inv, *scale_inv_used;
  int32_t *head, *status;
} state_t;

static void state_init(state_t* s) {
  const float one = 1.0f;
  HIP_OK(hipMalloc((void**)&s->history, L * sizeof(float)));
  HIP_OK(hipMalloc((void**)&s->amax, sizeof(float)));
  HIP_OK(hipMalloc((void**)&s->scale, sizeof(float)));
  HIP_OK(hipMalloc((void**)&s->scale_inv, sizeof(float)));
  HIP_OK(hipMalloc((void**)&s->scale_inv_used, sizeof(float)));
  HIP_OK(hipMalloc((void**)&s->head, sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&s->status, sizeof(int32_t)));
  HIP_OK(hipMemset(s->history, 0, L * sizeof(float)));
  HIP_OK(hipMemset(s->head, 0, sizeof(int32_t)));
  HIP_OK(hipMemset(s->status, 0, sizeof(int32_t)));
  HIP_OK(hipMemcpy(s->scale, &one, sizeof one, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(s->scale_inv, &one, sizeof one, hipMemcpyHostToDevice));
}

static void state_dump(const state_t* s, const char* dir, const char* name, int t) {
  unsigned char buf[4 * 4 + 2 * 4 + L * 4];
  float f[4];
  int32_t i[2];
  HIP_OK(hipMemcpy(&f[0], s->amax, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&f[1], s->scale, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&f[2], s->scale_inv, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&f[3], s->scale_inv_used, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&i[0], s->head, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&i[1], s->status, 4, hipMemcpyDeviceToHost));
  memcpy(buf, f, sizeof f);
  memcpy(buf + sizeof f, i, sizeof i);
  HIP_OK(hipMemcpy(buf + sizeof f + sizeof i, s->history, L * 4, hipMemcpyDeviceToHost));
  write_file(dir, name, t, buf, sizeof buf);
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUTDIR\n", argv[0]);
    return 1;
  }
  const char* dir = argv[1];
  uint16_t* hx = malloc((size_t)M * K * 2);
  uint16_t* hw = malloc((size_t)K * N * 2);
  uint8_t* hqx = malloc((size_t)M * K);
  uint8_t* hqwt = malloc((size_t)N * K);
  float* hc = malloc((size_t)M * N * 4);
  if (!hx || !hw || !hqx || !hqwt || !hc) return 1;

  void *x, *w, *ws, *c;
  uint8_t *qx, *qwt;
  HIP_OK(hipMalloc(&x, (size_t)M * K * 2));
  HIP_OK(hipMalloc(&w, (size_t)K * N * 2));
  HIP_OK(hipMalloc((void**)&qx, (size_t)M * K));
  HIP_OK(hipMalloc((void**)&qwt, (size_t)N * K));
  HIP_OK(hipMalloc(&c, (size_t)M * N * 4));
  HIP_OK(hipMalloc(&ws, FP8MI_QUANTIZE_WORKSPACE_BYTES));
  state_t sx, sw;
  state_init(&sx);
  state_init(&sw);

  for (int t = 0; t < STEPS; ++t) {
    /* The activations grow from step to step, so the delayed scale lags. */
    const float gx = 1.0f + 1.5f * (float)t, gw = 0.02f;
    for (size_t i = 0; i < (size_t)M * K; ++i) hx[i] = to_bf16(draw() * gx);
    for (size_t i = 0; i < (size_t)K * N; ++i) hw[i] = to_bf16(draw() * gw);
    HIP_OK(hipMemcpy(x, hx, (size_t)M * K * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(w, hw, (size_t)K * N * 2, hipMemcpyHostToDevice));
    /* X: row-major codes; W [K x N]: the transposed codes [N x K] the GEMM takes. */
    FP8_OK(fp8_quantize_update(x, FP8MI_BF16, M, K, FP8MI_E4M3, qx, NULL, sx.amax, NULL, ws,
                               FP8MI_QUANTIZE_WORKSPACE_BYTES, sx.history, L, sx.head, sx.scale, sx.scale_inv,
                               sx.status, sx.scale_inv_used, NULL));
    FP8_OK(fp8_quantize_update(w, FP8MI_BF16, K, N, FP8MI_E4M3, NULL, qwt, sw.amax, NULL, ws,
                               FP8MI_QUANTIZE_WORKSPACE_BYTES, sw.history, L, sw.head, sw.scale, sw.scale_inv,
                               sw.status, sw.scale_inv_used, NULL));
    FP8_OK(fp8_gemm(qx, FP8MI_E4M3, qwt, FP8MI_E4M3, 0, M, N, K, sx.scale_inv_used, sw.scale_inv_used, c, FP8MI_F32,
                    FP8MI_ACCUM_EXACT, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hqx, qx, (size_t)M * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hqwt, qwt, (size_t)N * K, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hc, c, (size_t)M * N * 4, hipMemcpyDeviceToHost));
    write_file(dir, "x", t, hx, (size_t)M * K * 2);
    write_file(dir, "w", t, hw, (size_t)K * N * 2);
    write_file(dir, "qx", t, hqx, (size_t)M * K);
    write_file(dir, "qwt", t, hqwt, (size_t)N * K);
    write_file(dir, "c", t, hc, (size_t)M * N * 4);
    state_dump(&sx, dir, "sx", t);
    state_dump(&sw, dir, "sw", t);
    printf("step %d done\n", t);
    fflush(stdout);
  }
  HIP_OK(hipFree(x));
  HIP_OK(hipFree(w));
  HIP_OK(hipFree(qx));
  HIP_OK(hipFree(qwt));
  HIP_OK(hipFree(c));
  HIP_OK(hipFree(ws));
  free(hx);
  free(hw);
  free(hqx);
  free(hqwt);
  free(hc);
  return 0;
}
