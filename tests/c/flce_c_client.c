/*
 * A plain C99 client of the FLCE C ABI (include/flce.h): links libflce.so and the HIP runtime,
 * with no C++ and no Python in the process.  Test infrastructure: the GPU and CPU tests run it.
 *
 *   flce_c_client host     calls that need no device: status strings, the automatic chunk rule,
 *                          argument errors on NULL handles and configurations.
 *   flce_c_client device   calls on the current HIP device with W = 0, where the method has a
 *                          closed form: every logit is 0, so lse = ln V, loss = ln V, dx = 0 and
 *                          dW[v] = (1/V) mean_n x_n - (1/N) sum_{n: t_n = v} x_n (the mean loss
 *                          and its gradient, with softmax = 1/V); fp32 and bf16 inputs, several
 *                          chunks with a ragged tail; then the argument and data errors.
 * Prints one line per check and "PASS <mode>" at the end; exits 1 on the first failure.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flce.h"

static int failures = 0;

#define CHECK(cond, ...)                    \
  do {                                      \
    if (!(cond)) {                          \
      printf("FAIL %s:%d: ", __FILE__, __LINE__); \
      printf(__VA_ARGS__);                  \
      printf("\n");                         \
      failures++;                           \
      return 1;                             \
    }                                       \
  } while (0)

#define HIP_OK(call) CHECK((call) == hipSuccess, "%s", #call)

static int host_mode(void) {
  const flce_status_t codes[] = {FLCE_OK, FLCE_ERR_INVALID_ARG, FLCE_ERR_UNSUPPORTED, FLCE_ERR_OOM,
                                 FLCE_ERR_HIP, FLCE_ERR_DATA};
  const char* names[] = {"FLCE_OK", "FLCE_ERR_INVALID_ARG", "FLCE_ERR_UNSUPPORTED", "FLCE_ERR_OOM",
                         "FLCE_ERR_HIP", "FLCE_ERR_DATA"};
  for (int i = 0; i < 6; ++i) {
    const char* s = flce_status_string(codes[i]);
    CHECK(s != NULL && strncmp(s, names[i], strlen(names[i])) == 0, "status string of %d", (int)codes[i]);
  }
  /* explicit chunks clamp to [1, N]; automatic ones follow the documented rule */
  CHECK(flce_effective_chunk(1000, 512, 5000, 384) == 384, "explicit chunk");
  CHECK(flce_effective_chunk(100, 512, 5000, 384) == 100, "chunk clamped to N");
  CHECK(flce_effective_chunk(16384, 4096, 128256, 0) == 4096, "automatic chunk, Llama-3 vocabulary");
  CHECK(flce_effective_chunk(0, 4096, 128256, 0) == 0, "invalid N gives 0");
  /* argument errors that are decided before any device work */
  flce_handle_t h = NULL;
  CHECK(flce_create(NULL, &h) == FLCE_ERR_INVALID_ARG, "NULL configuration");
  flce_config_t cfg;
  memset(&cfg, 0, sizeof(cfg));
  CHECK(flce_create(&cfg, NULL) == FLCE_ERR_INVALID_ARG, "NULL handle slot");
  CHECK(flce_destroy(NULL) == FLCE_OK, "destroy(NULL) is a no-op");
  float loss = 0.f;
  CHECK(flce_forward_backward(NULL, &loss, &loss, NULL, 1, 8, 2, 0, &loss, &loss, &loss, NULL) ==
            FLCE_ERR_INVALID_ARG, "NULL handle");
  CHECK(flce_workspace_bytes(NULL, 16, 8, 4, 0) == 0, "workspace of a NULL handle");
  CHECK(flce_check(NULL, NULL) == FLCE_ERR_INVALID_ARG, "check of a NULL handle");
  printf("PASS host\n");
  return 0;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
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
static float bf16_bits_to_float_at(const uint16_t* p, size_t i) { return from_bf16(p[i]); }

/* one W = 0 call against the closed form; bf16: inputs and outputs in bf16, else fp32 */
static int closed_form_case(int bf16, int64_t N, int64_t H, int64_t V, int64_t chunk, hipStream_t st) {
  const size_t es = bf16 ? 2 : 4;
  flce_config_t cfg;
  memset(&cfg, 0, sizeof(cfg));
  cfg.in_dtype = cfg.dx_dtype = cfg.dw_dtype = bf16 ? FLCE_BF16 : FLCE_FP32;
  cfg.variant = FLCE_CHUNKED;
  cfg.device = 0;
  flce_handle_t h = NULL;
  CHECK(flce_create(&cfg, &h) == FLCE_OK, "create");

  /* host inputs: x in [-1, 1) from a 64-bit LCG, rounded to the input dtype; targets spread */
  float* xf = (float*)malloc((size_t)(N * H) * sizeof(float));
  void* xh = malloc((size_t)(N * H) * es);
  int64_t* th = (int64_t*)malloc((size_t)N * sizeof(int64_t));
  uint64_t s = 0x9E3779B97F4A7C15ull;
  for (int64_t i = 0; i < N * H; ++i) {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    float v = (float)((double)(s >> 11) / 9007199254740992.0 * 2.0 - 1.0);
    if (bf16) {
      ((uint16_t*)xh)[i] = to_bf16(v);
      v = from_bf16(((uint16_t*)xh)[i]);
    } else {
      ((float*)xh)[i] = v;
    }
    xf[i] = v;
  }
  for (int64_t n = 0; n < N; ++n) th[n] = (n * 7919) % V;

  void *x, *W, *dx, *dW;
  int64_t* t;
  float *loss, *lse;
  HIP_OK(hipMalloc(&x, (size_t)(N * H) * es));
  HIP_OK(hipMalloc(&W, (size_t)(V * H) * es));
  HIP_OK(hipMalloc(&dx, (size_t)(N * H) * es));
  HIP_OK(hipMalloc(&dW, (size_t)(V * H) * es));
  HIP_OK(hipMalloc((void**)&t, (size_t)N * sizeof(int64_t)));
  HIP_OK(hipMalloc((void**)&loss, sizeof(float)));
  HIP_OK(hipMalloc((void**)&lse, (size_t)N * sizeof(float)));
  HIP_OK(hipMemcpy(x, xh, (size_t)(N * H) * es, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(W, 0, (size_t)(V * H) * es));
  HIP_OK(hipMemset(dx, 0x7f, (size_t)(N * H) * es));   /* overwritten by the call */
  HIP_OK(hipMemcpy(t, th, (size_t)N * sizeof(int64_t), hipMemcpyHostToDevice));
  CHECK(flce_reserve(h, N, H, V, chunk) == FLCE_OK, "reserve");
  CHECK(flce_forward_backward_ex(h, x, W, t, N, H, V, chunk, loss, dx, dW, lse, st) == FLCE_OK, "call");
  HIP_OK(hipStreamSynchronize(st));
  CHECK(flce_check(h, st) == FLCE_OK, "no data error");

  float lh = 0.f;
  float* lseh = (float*)malloc((size_t)N * sizeof(float));
  void* dxh = malloc((size_t)(N * H) * es);
  void* dWh = malloc((size_t)(V * H) * es);
  HIP_OK(hipMemcpy(&lh, loss, sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lseh, lse, (size_t)N * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dxh, dx, (size_t)(N * H) * es, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dWh, dW, (size_t)(V * H) * es, hipMemcpyDeviceToHost));

  const double lnV = log((double)V);
  CHECK(fabs(lh - lnV) <= 1e-5 * lnV, "loss %.8f, ln V %.8f", lh, lnV);
  for (int64_t n = 0; n < N; ++n) CHECK(fabs(lseh[n] - lnV) <= 1e-5 * lnV, "lse[%lld] %.8f", (long long)n, lseh[n]);
  for (int64_t i = 0; i < N * H; ++i) {
    const float v = bf16 ? bf16_bits_to_float_at((const uint16_t*)dxh, (size_t)i) : ((const float*)dxh)[i];
    CHECK(v == 0.f, "dx[%lld] = %g, not 0", (long long)i, v);
  }
  /* dW against its closed form, in fp64 */
  double* mean = (double*)calloc((size_t)H, sizeof(double));
  double* want = (double*)calloc((size_t)(V * H), sizeof(double));
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < H; ++k) mean[k] += xf[n * H + k] / (double)N;
  for (int64_t v = 0; v < V; ++v)
    for (int64_t k = 0; k < H; ++k) want[v * H + k] = mean[k] / (double)V;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < H; ++k) want[th[n] * H + k] -= xf[n * H + k] / (double)N;
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < V * H; ++i) {
    const double g = bf16 ? bf16_bits_to_float_at((const uint16_t*)dWh, (size_t)i) : ((const float*)dWh)[i];
    num += (g - want[i]) * (g - want[i]);
    den += want[i] * want[i];
  }
  const double rel = sqrt(num / den);
  /* bf16 output: each stored value rounds once per chunk (at most 2^-8 relative); fp32: ~1e-6 */
  const double tol = bf16 ? 2e-2 : 1e-5;
  CHECK(rel <= tol, "dW relative Frobenius error %.3e > %.1e", rel, tol);
  printf("ok  W = 0 closed form, %s, N=%lld H=%lld V=%lld chunk=%lld: loss %.7f, dW rel %.2e\n",
         bf16 ? "bf16" : "fp32", (long long)N, (long long)H, (long long)V, (long long)chunk, lh, rel);

  /* errors: invalid and unsupported arguments write nothing; a bad target raises the data flag */
  HIP_OK(hipMemset(dx, 0x7f, (size_t)(N * H) * es));
  CHECK(flce_forward_backward(h, x, W, t, 0, H, V, chunk, loss, dx, dW, st) == FLCE_ERR_INVALID_ARG, "N = 0");
  CHECK(flce_forward_backward(h, (const char*)x + 2, W, t, N, H, V, chunk, loss, dx, dW, st) == FLCE_ERR_UNSUPPORTED,
        "misaligned x");
  CHECK(flce_forward_backward(h, x, W, t, N, H + 4, V, chunk, loss, dx, dW, st) == FLCE_ERR_UNSUPPORTED, "H %% 8 != 0");
  CHECK(flce_forward_backward(h, x, W, t, N, H, V, chunk, loss, x, dW, st) == FLCE_ERR_INVALID_ARG, "dx over x");
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipMemcpy(dxh, dx, (size_t)(N * H) * es, hipMemcpyDeviceToHost));
  for (int64_t i = 0; i < N * H; ++i) CHECK(((const unsigned char*)dxh)[i * es] == 0x7f, "a refused call wrote dx");
  const int64_t bad = V + 5;
  HIP_OK(hipMemcpy(t + N / 2, &bad, sizeof(int64_t), hipMemcpyHostToDevice));
  CHECK(flce_forward_backward(h, x, W, t, N, H, V, chunk, loss, dx, dW, st) == FLCE_OK, "call with a bad target");
  CHECK(flce_check(h, st) == FLCE_ERR_DATA, "bad target reported");
  HIP_OK(hipMemcpy(&lh, loss, sizeof(float), hipMemcpyDeviceToHost));
  CHECK(isnan(lh), "loss with a bad target is NaN, got %g", lh);
  CHECK(flce_check(h, st) == FLCE_OK, "flag cleared by the check");
  printf("ok  errors: N = 0, misalignment, H %% 8, overlap, bad target\n");

  CHECK(flce_destroy(h) == FLCE_OK, "destroy");
  hipFree(x); hipFree(W); hipFree(dx); hipFree(dW); hipFree(t); hipFree(loss); hipFree(lse);
  free(xf); free(xh); free(th); free(lseh); free(dxh); free(dWh); free(mean); free(want);
  return 0;
}

static int device_mode(void) {
  int n = 0;
  HIP_OK(hipGetDeviceCount(&n));
  CHECK(n >= 1, "no HIP device");
  HIP_OK(hipSetDevice(0));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  if (closed_form_case(0, 300, 64, 1000, 128, st)) return 1;
  if (closed_form_case(1, 520, 136, 2100, 200, st)) return 1;
  HIP_OK(hipStreamDestroy(st));
  printf("PASS device\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "host") == 0) return host_mode() ? 1 : 0;
  if (argc == 2 && strcmp(argv[1], "device") == 0) return device_mode() ? 1 : 0;
  fprintf(stderr, "usage: %s host|device\n", argv[0]);
  return 2;
}
