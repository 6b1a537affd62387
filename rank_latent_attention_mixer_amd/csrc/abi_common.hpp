// Host-side helpers shared by the forward and backward halves of the C
// boundary (argument checks, workspace carving, the saved-tensor layout).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <initializer_list>

#include "../../include/flarepp.h"

namespace flarepp {

constexpr int kDecTargetWgs = 256;  // persistent token-pass workgroups (one per CU)
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

inline int esize_of(int dtype) { return dtype == FLAREPP_F32 ? 4 : 2; }


inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_mul_overflow(a, b, out);
}

// Shape checks shared by every entry point (no HIP call).
inline int check_shape(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype) {
  if (B < 1 || H < 1 || N < 1 || M < 1 || D < 1) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (dtype != FLAREPP_F32 && dtype != FLAREPP_BF16 && dtype != FLAREPP_F16)
    return FLAREPP_ERR_INVALID_ARGUMENT;
  int64_t t;
  if (!mul_ok(B, H, &t) || !mul_ok(t, N, &t) || !mul_ok(t, D, &t) || !mul_ok(t, 4, &t))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  if (!mul_ok(H, M, &t) || !mul_ok(t, D, &t)) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (B * H > (int64_t)1 << 24) return FLAREPP_ERR_INVALID_ARGUMENT;  // grid limits
  if (D != 8 && D != 16 && D != 32 && D != 64) return FLAREPP_ERR_UNSUPPORTED;
  if (M > FLAREPP_MAX_M) return FLAREPP_ERR_UNSUPPORTED;
  return FLAREPP_OK;
}


inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}


inline int hip_status(hipError_t e) { return e == hipSuccess ? FLAREPP_OK : FLAREPP_ERR_HIP; }

inline unsigned char* ws_at(void* ws, size_t off) { return static_cast<unsigned char*>(ws) + off; }


struct Saved {
  float *q, *z, *qd, *lse0, *lse1, *lse2;
  size_t floats;
};
// base may be null (a forward that saves nothing): then every slot is null
// and only `floats` is meaningful (no arithmetic on a null pointer)
inline Saved saved_layout(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, float* base) {
  Saved v;
  const size_t lat = (size_t)(B * H * M * D), row = (size_t)(B * H * M);
  size_t o = 0;
  auto at = [base](size_t off) { return base ? base + off : nullptr; };
  v.q = at(o); o += lat;
  v.z = at(o); o += lat;
  v.qd = at(o); o += lat;
  v.lse0 = at(o); o += row;
  v.lse1 = at(o); o += row;
  v.lse2 = at(o); o += (size_t)(B * H * N);
  v.floats = o;
  return v;
}


#define FLAREPP_TRY(expr)                        \
  do {                                           \
    const hipError_t e_ = (expr);                \
    if (e_ != hipSuccess) return FLAREPP_ERR_HIP; \
  } while (0)

// A caller buffer: address and bytes (null or empty: not present).
struct Span {
  const void* p;
  size_t n;
};

// True if an output buffer overlaps another output or any input (inputs
// include the workspace and saved tensors).  Outputs are written by the
// kernels, so any such overlap would corrupt a result.
inline bool outputs_alias(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    if (!o->p || !o->n) continue;
    for (auto q = o + 1; q != outs.end(); ++q)
      if (q->p && q->n && overlaps(o->p, o->n, q->p, q->n)) return true;
    for (const Span& i : ins)
      if (i.p && i.n && overlaps(o->p, o->n, i.p, i.n)) return true;
  }
  return false;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// gfx950 check for the current device, cached per device id.
int check_device();

}  // namespace flarepp
