// Instruction-throughput probes of the two units the mixer's kernels are
// bound by: the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) and the
// transcendental rate (v_exp_f32), and how much vector-ALU work the matrix
// cores hide on one SIMD.  Measurement infrastructure for the
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

// The matrix cores' sustained rate depends on the data they multiply: the
// chip's power limit lowers the clock further when the operand bits toggle.
// Both variants issue the same products (four independent accumulators,
// operands rotating through eight registers); RANDOM fills the operands with
// hashed bf16 values of random sign and mantissa in [1, 2) (the toggling of
// real activations), the other with 1.0 everywhere.
__device__ __forceinline__ unsigned probe_hash(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <bool RANDOM>
__global__ __launch_bounds__(256) void mfma_data_probe(float* out, int iters) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  bf16x8 r[8];
  for (int j = 0; j < 8; ++j) {
    u32x4 t;
    for (int e = 0; e < 4; ++e) {
      const unsigned h = probe_hash((blockIdx.x * 256u + threadIdx.x) * 37u + j * 5u + e);
      const unsigned lo = 0x3F80u | (h & 0x807Fu), hi = 0x3F80u | ((h >> 16) & 0x807Fu);
      t[e] = RANDOM ? (lo | (hi << 16)) : 0x3F803F80u;
    }
    r[j] = __builtin_bit_cast(bf16x8, t);
  }
  f32x16 c[4];
  for (int j = 0; j < 4; ++j)
    for (int v = 0; v < 16; ++v) c[j][v] = 0.f;
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[(u + j) & 7], r[(u + 2 * j + 1) & 7], c[j],
                                                        0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int v = 0; v < 16; ++v) s += c[j][v];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Co-issue of the vector ALU with the matrix cores on one SIMD: per
// iteration, four independent 32x32x16 products (MFMA), 32 independent
// fp32 FMAs with three register sources (FMA), or both (MIX, each product
// followed by eight FMAs in the instruction stream).  The three times give
// the share of the FMA time that the products hide.
template <bool MF, bool FM>
__global__ __launch_bounds__(256) void coissue_probe(float* out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  float x[16], y[16], z[16];
  for (int i = 0; i < 16; ++i) {
    x[i] = seed * (float)(lane + i);
    y[i] = 0.999f + 1e-6f * (float)(lane ^ i);
    z[i] = 1e-3f * (float)(i + lane);
  }
  bf16x8 a;
  for (int i = 0; i < 8; ++i) a[i] = (__bf16)(seed * (float)(lane + i + 1));
  f32x16 c[4];
  for (int j = 0; j < 4; ++j)
    for (int v = 0; v < 16; ++v) c[j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
    if constexpr (MF) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c[j], 0, 0, 0);
    }
    if constexpr (FM) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], y[i], z[i]);
    }
    if constexpr (MF && FM) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // eight VALU
      }
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += x[i];
  for (int j = 0; j < 4; ++j) s += c[j][lane & 15];
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
  else if (which == FLAREPP_PROBE_MFMA_BF16_RANDOM)
    hipLaunchKernelGGL(mfma_data_probe<true>, dim3(blocks), dim3(256), 0, s, out, iters);
  else if (which == FLAREPP_PROBE_MFMA_BF16_ONES)
    hipLaunchKernelGGL(mfma_data_probe<false>, dim3(blocks), dim3(256), 0, s, out, iters);
  else if (which == FLAREPP_PROBE_COISSUE_MFMA)
    hipLaunchKernelGGL((coissue_probe<true, false>), dim3(blocks), dim3(256), 0, s, out, iters, 1e-3f);
  else if (which == FLAREPP_PROBE_COISSUE_FMA)
    hipLaunchKernelGGL((coissue_probe<false, true>), dim3(blocks), dim3(256), 0, s, out, iters, 1e-3f);
  else if (which == FLAREPP_PROBE_COISSUE_MIX)
    hipLaunchKernelGGL((coissue_probe<true, true>), dim3(blocks), dim3(256), 0, s, out, iters, 1e-3f);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

double flarepp_probe_work(int which, int blocks, int iters) {
  const double lanes = 256.0 * blocks;
  if (which == FLAREPP_PROBE_MFMA_BF16)  // per wave: iters x 8 products of 2*32*32*16 flops
    return (lanes / 64.0) * iters * 8.0 * 2.0 * 32 * 32 * 16;
  if (which == FLAREPP_PROBE_EXP_F32) return lanes * iters * 8.0;  // exponentials
  if (which == FLAREPP_PROBE_MFMA_BF16_RANDOM || which == FLAREPP_PROBE_MFMA_BF16_ONES)
    return (lanes / 64.0) * ((iters + 7) / 8 * 8) * 4.0 * 2.0 * 32 * 32 * 16;
  if (which >= FLAREPP_PROBE_COISSUE_MFMA && which <= FLAREPP_PROBE_COISSUE_MIX)
    return (lanes / 64.0) * iters;  // wave-iterations
  return 0.0;
}

}  // extern "C"
