// Parameters and launchers of the front-end kernels (frontend.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace flarepp {

// Three head-split projections of the tokens, k0 normalised head-wise.
struct FrontendParams {
  const void* x;          // [T, C] dtype, T = B N tokens
  const void* w[3];       // [H D, C] dtype: k0, k, v
  const void* b[3];       // [H D] dtype or null
  const void* g;          // [H, D] dtype gain of the k0 normalisation, or null (1)
  void* out[3];           // [B, H, N, D] dtype: k0, k, v
  int64_t T, N, C;
  int H;
  int normalize;          // 0: k0 as projected
  float eps;
};

// Head-wise normalisation of the seeds q0 [H, M, D].
struct SeedNormParams {
  const void* q0;
  const void* g;          // [H, D] or null
  void* out;
  int H, M, D;
  float eps;
};

hipError_t launch_frontend(int dtype, int D, const FrontendParams& p, hipStream_t s);
hipError_t launch_seed_norm(int dtype, const SeedNormParams& p, hipStream_t s);

}  // namespace flarepp
