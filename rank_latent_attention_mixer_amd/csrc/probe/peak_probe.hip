// Instruction-throughput probes of the two units the mixer's kernels are
// bound by: the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) and the
// transcendental rate (v_exp_f32).  Measurement infrastructure for the
// roofline (the measured peak beside the published one); not part of the
// mixer's C boundary.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../../include/flarepp_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Eight independent accumulator chains per wave keep the matrix core busy
// without dependency stalls; the result is written so nothing folds away.
__global__ __launch_bounds__(256) void mfma_probe(float* out, int iters, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(i + 1));
    b[i] = (__bf16)(seed * (float)(threadIdx.x + i));
  }
  f32x16 c[8];
  for (int j = 0; j < 8; ++j)
    for (int v = 0; v < 16; ++v) c[j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int v = 0; v < 16; ++v) s += c[j][v];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Eight independent exp chains per lane.
__global__ __launch_bounds__(256) void exp_probe(float* out, int iters, float seed) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = -seed * (float)(threadIdx.x + i) * 1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int flarepp_probe_launch(int which, int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (which == FLAREPP_PROBE_MFMA_BF16)
    hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(256), 0, s, out, iters, 1e-3f);
  else if (which == FLAREPP_PROBE_EXP_F32)
    hipLaunchKernelGGL(exp_probe, dim3(blocks), dim3(256), 0, s, out, iters, 1e-3f);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

double flarepp_probe_work(int which, int blocks, int iters) {
  const double lanes = 256.0 * blocks;
  if (which == FLAREPP_PROBE_MFMA_BF16)  // per wave: iters x 8 products of 2*32*32*16 flops
    return (lanes / 64.0) * iters * 8.0 * 2.0 * 32 * 32 * 16;
  if (which == FLAREPP_PROBE_EXP_F32) return lanes * iters * 8.0;  // exponentials
  return 0.0;
}

}  // extern "C"
