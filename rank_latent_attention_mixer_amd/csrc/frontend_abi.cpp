// C boundary of the front end: argument validation and launch of the
// projection and seed-normalisation kernels (include/flarepp.h).
#include <cmath>
#include <cstring>

#include "abi_common.hpp"
#include "frontend.hpp"

using namespace flarepp;

namespace {

int check_frontend_shape(int64_t B, int64_t N, int64_t C, int64_t H, int64_t D, int dtype) {
  if (B < 1 || N < 1 || C < 1 || H < 1 || D < 1) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (dtype != FLAREPP_F32 && dtype != FLAREPP_BF16 && dtype != FLAREPP_F16)
    return FLAREPP_ERR_INVALID_ARGUMENT;
  int64_t t;
  if (!mul_ok(B, N, &t) || !mul_ok(t, C, &t) || !mul_ok(t, 2, &t)) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (!mul_ok(B, H, &t) || !mul_ok(t, N, &t) || !mul_ok(t, D, &t) || !mul_ok(t, 2, &t))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  if (!mul_ok(H, D, &t) || !mul_ok(t, 3 * C, &t)) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (dtype == FLAREPP_F32) return FLAREPP_ERR_UNSUPPORTED;  // matrix-core path only
  if (D != 16 && D != 32 && D != 64) return FLAREPP_ERR_UNSUPPORTED;
  if (C % 16 != 0) return FLAREPP_ERR_UNSUPPORTED;
  if (H > (1 << 20)) return FLAREPP_ERR_UNSUPPORTED;
  return FLAREPP_OK;
}

}  // namespace

extern "C" {

int flarepp_frontend_fwd(int64_t B, int64_t N, int64_t C, int64_t H, int64_t D, int dtype,
                         const void* x, const void* w_k0, const void* w_k, const void* w_v,
                         const void* b_k0, const void* b_k, const void* b_v, const void* g_k0,
                         float eps, int normalize_k0, void* k0, void* k, void* v, void* stream) {
  try {
    int st = check_frontend_shape(B, N, C, H, D, dtype);
    if (st != FLAREPP_OK) return st;
    if (!x || !w_k0 || !w_k || !w_v || !k0 || !k || !v) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (normalize_k0 && !(std::isfinite(eps) && eps > 0.f)) return FLAREPP_ERR_INVALID_ARGUMENT;
    for (const void* p : {x, w_k0, w_k, w_v, (const void*)k0, (const void*)k, (const void*)v})
      if (!aligned16(p)) return FLAREPP_ERR_INVALID_ARGUMENT;
    const size_t e = 2;
    const size_t xb = (size_t)(B * N * C) * e, wb = (size_t)(H * D * C) * e;
    const size_t ob = (size_t)(B * H * N * D) * e, bb = (size_t)(H * D) * e;
    void* outs[3] = {k0, k, v};
    for (int i = 0; i < 3; ++i) {
      for (int j = i + 1; j < 3; ++j)
        if (overlaps(outs[i], ob, outs[j], ob)) return FLAREPP_ERR_INVALID_ARGUMENT;
      if (overlaps(outs[i], ob, x, xb)) return FLAREPP_ERR_INVALID_ARGUMENT;
      for (const void* w : {w_k0, w_k, w_v})
        if (overlaps(outs[i], ob, w, wb)) return FLAREPP_ERR_INVALID_ARGUMENT;
      for (const void* b : {b_k0, b_k, b_v, g_k0})
        if (b && overlaps(outs[i], ob, b, bb)) return FLAREPP_ERR_INVALID_ARGUMENT;
    }
    if ((st = check_device()) != FLAREPP_OK) return st;
    FrontendParams p;
    std::memset(&p, 0, sizeof(p));
    p.x = x;
    p.w[0] = w_k0; p.w[1] = w_k; p.w[2] = w_v;
    p.b[0] = b_k0; p.b[1] = b_k; p.b[2] = b_v;
    p.g = g_k0;
    p.out[0] = k0; p.out[1] = k; p.out[2] = v;
    p.T = B * N; p.N = N; p.C = C; p.H = (int)H;
    p.normalize = normalize_k0 ? 1 : 0;
    p.eps = eps;
    return hip_status(launch_frontend(dtype, (int)D, p, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int flarepp_seed_norm_fwd(int64_t H, int64_t M, int64_t D, int dtype, const void* q0,
                          const void* g_q0, float eps, void* q0_out, void* stream) {
  try {
    if (H < 1 || M < 1 || D < 1 || !q0 || !q0_out) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (dtype != FLAREPP_BF16 && dtype != FLAREPP_F16)
      return dtype == FLAREPP_F32 ? FLAREPP_ERR_UNSUPPORTED : FLAREPP_ERR_INVALID_ARGUMENT;
    if (D > 64 || H * M > ((int64_t)1 << 30)) return FLAREPP_ERR_UNSUPPORTED;
    if (!(std::isfinite(eps) && eps > 0.f)) return FLAREPP_ERR_INVALID_ARGUMENT;
    const size_t n = (size_t)(H * M * D) * 2;
    // in place (q0_out == q0) is allowed: a row is read whole before it is written
    if ((q0_out != q0 && overlaps(q0_out, n, q0, n)) ||
        (g_q0 && overlaps(q0_out, n, g_q0, (size_t)(H * D) * 2)))
      return FLAREPP_ERR_INVALID_ARGUMENT;
    int st;
    if ((st = check_device()) != FLAREPP_OK) return st;
    SeedNormParams p;
    p.q0 = q0; p.g = g_q0; p.out = q0_out;
    p.H = (int)H; p.M = (int)M; p.D = (int)D; p.eps = eps;
    return hip_status(launch_seed_norm(dtype, p, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

}  // extern "C"
