/* A plain-C client of libflarepp (no Python, no torch): device memory from
 * the HIP runtime, the mixer through its C entry points, on small cases
 * whose outputs follow in closed form from the definition of the mixer
 * (FLARE.py README, "FLARE++" and "FLARE" listings: softmax attentions over
 * the keys), plus one argument error.  Built next to this file by the
 * package build; run by tests/test_gpu_c_abi.py.  Prints one line per check
 * and exits 0 when all pass. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flarepp.h"

static int failures = 0;

#define HIP_OK(x)                                                      \
  do {                                                                 \
    hipError_t e_ = (x);                                               \
    if (e_ != hipSuccess) {                                            \
      printf("hip error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                         \
    }                                                                  \
  } while (0)

static float* to_device(const float* h, size_t n) {
  float* d = NULL;
  HIP_OK(hipMalloc((void**)&d, n * sizeof(float) + 16));
  HIP_OK(hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice));
  return d;
}

static void check(const char* what, double err, double bar) {
  const int ok = err <= bar;
  printf("%s %s: max error %.3e (bar %.1e)\n", ok ? "ok" : "FAIL", what, err, bar);
  if (!ok) ++failures;
}

/* deterministic values in [-1, 1) */
static float lcg(unsigned* s) {
  *s = *s * 1664525u + 1013904223u;
  return (float)((*s >> 8) & 0xFFFF) / 32768.0f - 1.0f;
}

/* y of flarepp_mixer_fwd in fp32 for the given host tensors */
static int run_flarepp(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, const float* q0,
                       const float* qf, const float* gate, const float* k0, const float* k,
                       const float* v, float* y) {
  const size_t lat = (size_t)(H * M * D), tok = (size_t)(B * H * N * D);
  float *dq0 = to_device(q0, lat), *dqf = to_device(qf, lat), *dg = to_device(gate, (size_t)H);
  float *dk0 = to_device(k0, tok), *dk = to_device(k, tok), *dv = to_device(v, tok);
  float* dy = NULL;
  void* ws = NULL;
  HIP_OK(hipMalloc((void**)&dy, tok * sizeof(float)));
  const size_t wsb = flarepp_workspace_size(B, H, N, M, D, FLAREPP_F32);
  HIP_OK(hipMalloc(&ws, wsb));
  const int st = flarepp_mixer_fwd(B, H, N, M, D, FLAREPP_F32, dq0, dqf, dg, dk0, dk, dv, dy, ws,
                                   wsb, NULL);
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(y, dy, tok * sizeof(float), hipMemcpyDeviceToHost));
  hipFree(dq0); hipFree(dqf); hipFree(dg); hipFree(dk0); hipFree(dk); hipFree(dv); hipFree(dy);
  hipFree(ws);
  return st;
}

int main(void) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    printf("no device\n");
    return 3;
  }
  printf("libflarepp %s\n", flarepp_version());
  const int64_t B = 2, H = 3, M = 16, D = 32;
  unsigned seed = 12345u;
  for (int c = 0; c < 2; ++c) {
    /* case 0: a single token -- every softmax over the keys has one entry,
     * so y = v whatever the latents and gates.  case 1: gate closed and
     * q_fixed = 0 -- the encoder's scores are all 0, z = mean_n v, and y = z. */
    const int64_t N = c == 0 ? 1 : 200;
    const size_t lat = (size_t)(H * M * D), tok = (size_t)(B * H * N * D);
    float* q0 = malloc(lat * sizeof(float));
    float* qf = malloc(lat * sizeof(float));
    float* k0 = malloc(tok * sizeof(float));
    float* k = malloc(tok * sizeof(float));
    float* v = malloc(tok * sizeof(float));
    float* y = malloc(tok * sizeof(float));
    float gate[3];
    for (size_t i = 0; i < lat; ++i) { q0[i] = lcg(&seed); qf[i] = c == 0 ? lcg(&seed) : 0.f; }
    for (size_t i = 0; i < tok; ++i) { k0[i] = lcg(&seed); k[i] = lcg(&seed); v[i] = lcg(&seed); }
    for (int h = 0; h < 3; ++h) gate[h] = c == 0 ? 0.5f * (float)h - 0.5f : -INFINITY;
    const int st = run_flarepp(B, H, N, M, D, q0, qf, gate, k0, k, v, y);
    if (st != FLAREPP_OK) {
      printf("FAIL flarepp_mixer_fwd returned %d (%s)\n", st, flarepp_status_string(st));
      ++failures;
    } else {
      double err = 0.0;
      for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t d = 0; d < D; ++d) {
          double mean = 0.0;
          for (int64_t n = 0; n < N; ++n) mean += v[(bh * N + n) * D + d];
          mean /= (double)N;
          for (int64_t n = 0; n < N; ++n) {
            const double e = fabs((double)y[(bh * N + n) * D + d] - mean);
            if (e > err) err = e;
          }
        }
      check(c == 0 ? "single token: y = v" : "closed gate, q_fixed = 0: y = mean_n v", err, 1e-5);
    }
    free(q0); free(qf); free(k0); free(k); free(v); free(y);
  }
  /* an argument error is reported before any launch */
  {
    const int st = flarepp_mixer_fwd(1, 1, 4, 4, 32, FLAREPP_F32, NULL, NULL, NULL, NULL, NULL, NULL,
                                     NULL, NULL, 0, NULL);
    const int ok = st == FLAREPP_ERR_INVALID_ARGUMENT && strlen(flarepp_status_string(st)) > 0;
    printf("%s null arguments: status %d (%s)\n", ok ? "ok" : "FAIL", st, flarepp_status_string(st));
    if (!ok) ++failures;
  }
  printf(failures ? "FAILED %d\n" : "all passed\n", failures);
  return failures ? 1 : 0;
}
