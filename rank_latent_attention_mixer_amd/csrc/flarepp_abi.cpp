// C boundary of libflarepp: argument validation, workspace carving and the
// launch sequence of each entry point.  See include/flarepp.h for the
// contract (the operations are those of the FLARE.py README, "FLARE++" and
// "FLARE" listings, with the gate of issue #2024 "Changes from v1 to v2").
#include "../../include/flarepp.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "abi_common.hpp"
#include "kernels.hpp"

namespace flarepp {

// gfx950 check for the current device, cached per device id.
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FLAREPP_ERR_HIP;
  if (dev < 64) {
    const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return FLAREPP_OK;
    if (c == 2) return FLAREPP_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FLAREPP_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FLAREPP_OK : FLAREPP_ERR_UNSUPPORTED;
}

}  // namespace flarepp

namespace {

using namespace flarepp;

constexpr int kEncTile = 64;        // granularity of caller-chosen encoder chunks
// encoder workgroups aimed for: one round of resident workgroups.  A 16-wave
// workgroup (M > 256) holds a CU alone; the smaller ones fit two per CU.
// Measured at the million-token shape: 256 workgroups of 16 waves 0.8%
// faster than 512 (half the chunk partials to merge); at the wide-head
// shape (4 waves) 256 was 20% slower than 512.
inline int64_t enc_target_wgs(int64_t M, int dtype) {
  return (dtype != FLAREPP_F32 && encode_waves((int)M) >= 16) ? 256 : 512;
}
struct Plan {
  int64_t B, H, N, M, D;
  int dtype;
  int Mpad;
  int64_t chunk_tokens;
  int nchunks;
  int dec_wg_per_bh;
  size_t off_pm, off_pl, off_po, off_q, off_z, off_redo, total;
};

int make_plan(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
              int64_t chunk_tokens, Plan* p) {
  int st = check_shape(B, H, N, M, D, dtype);
  if (st != FLAREPP_OK) return st;
  if (chunk_tokens < 0 || (chunk_tokens % kEncTile) != 0) return FLAREPP_ERR_INVALID_ARGUMENT;
  p->B = B; p->H = H; p->N = N; p->M = M; p->D = D; p->dtype = dtype;
  p->Mpad = latent_pad((int)M, dtype);
  const int64_t BH = B * H;
  if (chunk_tokens == 0) {
    // automatic chunks: whole encoder tiles, about enc_target_wgs workgroups
    const int64_t unit = dtype == FLAREPP_F32 ? kEncTile : encode_tile_tokens();
    const int64_t tiles = (N + unit - 1) / unit;
    const int64_t target = enc_target_wgs(M, dtype);
    int64_t c = (target + BH - 1) / BH;
    if (c < 1) c = 1;
    if (c > tiles) c = tiles;
    const int64_t chunk_tiles = (tiles + c - 1) / c;
    chunk_tokens = chunk_tiles * unit;
  }
  const int64_t nchunks = (N + chunk_tokens - 1) / chunk_tokens;
  int64_t wgs;
  if (!mul_ok(BH, nchunks, &wgs) || wgs > 0x7FFFFFFF) return FLAREPP_ERR_INVALID_ARGUMENT;
  p->chunk_tokens = chunk_tokens;
  p->nchunks = (int)nchunks;
  const int64_t dtiles = (N + decode_tokens_per_tile((int)D) - 1) / decode_tokens_per_tile((int)D);
  int64_t w = (kDecTargetWgs + BH - 1) / BH;
  if (w > dtiles) w = dtiles;
  if (w < 1) w = 1;
  p->dec_wg_per_bh = (int)w;
  if (!mul_ok(BH, w, &wgs) || wgs > 0x7FFFFFFF) return FLAREPP_ERR_INVALID_ARGUMENT;

  const size_t es = (size_t)esize_of(dtype);
  const size_t stat = (size_t)BH * nchunks * p->Mpad * sizeof(float);
  size_t off = 0;
  p->off_pm = off; off = align_up(off + stat);
  p->off_pl = off; off = align_up(off + stat);
  p->off_po = off; off = align_up(off + stat * D);
  p->off_q = off;  off = align_up(off + (size_t)BH * p->Mpad * D * es);
  p->off_z = off;  // value operand, natural [Mpad][D] rows (fp32 on the fp32 path)
  off = align_up(off + (size_t)BH * p->Mpad * D * (dtype == FLAREPP_F32 ? 4 : es));
  // decoder: per (workgroup, wave) record of tiles needing the exact path
  p->off_redo = off;
  off = align_up(off + (size_t)BH * w * decode_waves((int)D) * 2 * sizeof(unsigned long long));
  p->total = off;
  return FLAREPP_OK;
}

int check_workspace(const Plan& p, void* ws, size_t bytes) {
  if (ws == nullptr || bytes < p.total || ((uintptr_t)ws % kAlign) != 0)
    return FLAREPP_ERR_WORKSPACE;
  return FLAREPP_OK;
}

// qscale > 0: q is the caller's latents [.., M, D]; the kernel forms the
// operand (dtype)(qscale q) as it loads them.  0: q is an operand the
// combine kernel wrote ([.., Mpad, D], prescaled).
EncodeParams encode_params(const Plan& p, void* ws, const void* q, int64_t qb, int64_t qh,
                           const void* k, const void* v, const float* gate, float qscale = 0.f) {
  EncodeParams e;
  e.q = q; e.q_b_stride = qb; e.q_h_stride = qh; e.qscale = qscale;
  e.k = k; e.v = v;
  e.B = (int)p.B; e.H = (int)p.H; e.N = p.N; e.M = (int)p.M; e.Mpad = p.Mpad;
  e.chunk_tokens = p.chunk_tokens; e.nchunks = p.nchunks;
  e.gate = gate;
  e.part_m = reinterpret_cast<float*>(ws_at(ws, p.off_pm));
  e.part_l = reinterpret_cast<float*>(ws_at(ws, p.off_pl));
  e.part_o = reinterpret_cast<float*>(ws_at(ws, p.off_po));
  return e;
}

// Tensors a training forward saves for the backward pass (fp32, natural
// layouts): q [B,H,M,D] (the routing query), z [B,H,M,D], q_dyn [B,H,M,D],
// base-2 log-sum-exp of the synthesis and encoder rows [B,H,M] and of the
// decoder rows [B,H,N].
CombineParams combine_base(const Plan& p, void* ws) {
  CombineParams c;
  std::memset(&c, 0, sizeof(c));
  c.B = (int)p.B; c.H = (int)p.H; c.M = (int)p.M; c.Mpad = p.Mpad; c.D = (int)p.D;
  c.part_m = reinterpret_cast<const float*>(ws_at(ws, p.off_pm));
  c.part_l = reinterpret_cast<const float*>(ws_at(ws, p.off_pl));
  c.part_o = reinterpret_cast<const float*>(ws_at(ws, p.off_po));
  c.out_dtype = p.dtype;
  return c;
}

hipError_t value_operand(const Plan& p, void* ws, int nchunks, const float* z_in, float* z_out,
                         hipStream_t s, float* lse_out = nullptr) {
  CombineParams c = combine_base(p, ws);
  c.nsets = (int)(p.B * p.H);
  c.nchunks = nchunks;
  c.mode = kModeValue;
  c.z_in = z_in;
  c.z_out = z_out;
  c.lse_out = lse_out;
  c.out = ws_at(ws, p.off_z);
  c.out_kind = p.dtype == FLAREPP_F32 ? kOutNatural32 : kOutNatural;
  return launch_combine(c, s);
}

hipError_t decode(const Plan& p, void* ws, const void* q, int64_t qb, int64_t qh, const void* k,
                  void* y, hipStream_t s, float* lse_out = nullptr, float qscale = 0.f) {
  DecodeParams d;
  d.lse_out = lse_out;
  d.q = q; d.q_b_stride = qb; d.q_h_stride = qh; d.qscale = qscale;
  d.zt = ws_at(ws, p.off_z);
  d.redo = reinterpret_cast<unsigned long long*>(ws_at(ws, p.off_redo));
  d.k = k; d.y = y;
  d.B = (int)p.B; d.H = (int)p.H; d.N = p.N; d.M = (int)p.M; d.Mpad = p.Mpad;
  d.wg_per_bh = p.dec_wg_per_bh;
  return launch_decode(p.dtype, (int)p.D, d, s);
}

// Storage of the allocation-free forward: one array per device, owned by the
// library for the life of the process.  Host code never uses the array's
// name as an address: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[FLAREPP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FLAREPP_ERR_HIP;
  if (dev >= kMaxDevices) return FLAREPP_ERR_UNSUPPORTED;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return FLAREPP_ERR_HIP;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return FLAREPP_OK;
}

// FLARE++ (v0 == k0, q_fixed and gate given) and simplified FLARE++ (own
// synthesis values v0, q_fixed == gate == NULL: q is the synthesized query).
int mixer_impl(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, const void* q0,
               const void* q_fixed, const float* gate, const void* k0, const void* v0,
               const void* k, const void* v, void* y, void* ws, size_t ws_bytes, void* stream,
               void* const* events, float* saved = nullptr, size_t saved_bytes = 0,
               bool scratch_ws = false) {
  const bool simplified = q_fixed == nullptr && gate == nullptr;
  if (!q0 || !k0 || !v0 || !k || !v || !y) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (!aligned16(q0) || !aligned16(k0) || !aligned16(v0) || !aligned16(k) || !aligned16(v) ||
      !aligned16(y) || (q_fixed && !aligned16(q_fixed)))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  Plan p;
  int st = make_plan(B, H, N, M, D, dtype, 0, &p);
  if (st != FLAREPP_OK) return st;
  const size_t tok = (size_t)(B * H * N * D) * esize_of(dtype);
  const size_t lat = (size_t)(H * M * D) * esize_of(dtype);
  if (overlaps(y, tok, k0, tok) || overlaps(y, tok, v0, tok) || overlaps(y, tok, k, tok) ||
      overlaps(y, tok, v, tok) || overlaps(y, tok, q0, lat) ||
      (!simplified && (overlaps(y, tok, q_fixed, lat) || overlaps(y, tok, gate, (size_t)H * 4))))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  // scratch_ws: the library's own per-device array instead of a caller
  // workspace (its size was checked by the caller; no caller buffer can
  // overlap it); its address is taken after the device check
  if (scratch_ws) {
    if (p.total > ws_bytes) return FLAREPP_ERR_WORKSPACE;
  } else if ((st = check_workspace(p, ws, ws_bytes)) != FLAREPP_OK) {
    return st;
  }
  Saved sv = saved_layout(B, H, N, M, D, saved);
  if (saved && (saved_bytes < sv.floats * sizeof(float) ||
                (reinterpret_cast<uintptr_t>(saved) & 15)))
    return FLAREPP_ERR_WORKSPACE;
  if (outputs_alias({{y, tok}, {saved, saved ? sv.floats * 4 : 0},
                     {ws, scratch_ws ? 0 : ws_bytes}},
                    {{q0, lat}, {q_fixed, lat}, {gate, gate ? (size_t)H * 4 : 0}, {k0, tok},
                     {v0, tok}, {k, tok}, {v, tok}}))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  if ((st = check_device()) != FLAREPP_OK) return st;
  if (scratch_ws && (st = scratch_for_current_device(&ws)) != FLAREPP_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const float c = (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634);
  const int64_t BH = B * H;
  const int64_t qh = (int64_t)p.Mpad * D;
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : hipSuccess;
  };
  FLAREPP_TRY(mark(0));
  // 1. synthesis partials (closed-gate heads skipped); the seeds are scaled
  // as the encoder loads them, so nothing runs between marks 0 and 1
  FLAREPP_TRY(mark(1));
  FLAREPP_TRY(launch_encode(dtype, (int)D,
                            encode_params(p, ws, q0, 0, M * D, k0, v0, gate, c), s));
  FLAREPP_TRY(mark(2));
  // 3. q = q_fixed + sigma * q_dyn (simplified: q = q_dyn), per (b, h), as operand
  {
    CombineParams cp = combine_base(p, ws);
    cp.nsets = (int)BH;
    cp.nchunks = p.nchunks;
    cp.mode = kModeQuery;
    cp.fixed = q_fixed;
    cp.fixed_b_stride = 0;
    cp.fixed_dtype = dtype;
    cp.gate = gate;
    cp.cscale = c;
    cp.out = ws_at(ws, p.off_q);
    cp.out_kind = dtype == FLAREPP_F32 ? kOutNatural32 : kOutNatural;
    if (saved) {
      cp.q_out = sv.q;
      cp.dyn_out = sv.qd;
      cp.lse_out = sv.lse0;
    }
    FLAREPP_TRY(launch_combine(cp, s));
  }
  FLAREPP_TRY(mark(3));
  // 4. encode partials, 5. z as value operand, 6. decode
  FLAREPP_TRY(launch_encode(dtype, (int)D,
                            encode_params(p, ws, ws_at(ws, p.off_q), H * qh, qh, k, v, nullptr),
                            s));
  FLAREPP_TRY(mark(4));
  FLAREPP_TRY(value_operand(p, ws, p.nchunks, nullptr, saved ? sv.z : nullptr, s,
                            saved ? sv.lse1 : nullptr));
  FLAREPP_TRY(mark(5));
  FLAREPP_TRY(decode(p, ws, ws_at(ws, p.off_q), H * qh, qh, k, y, s, saved ? sv.lse2 : nullptr));
  FLAREPP_TRY(mark(6));
  return FLAREPP_OK;
}

int flare_impl(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, float scale,
               const void* q, const void* k, const void* v, void* y, void* ws, size_t ws_bytes,
               void* stream, float* saved = nullptr, size_t saved_bytes = 0) {
  if (!q || !k || !v || !y) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  Plan p;
  int st = make_plan(B, H, N, M, D, dtype, 0, &p);
  if (st != FLAREPP_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FLAREPP_ERR_INVALID_ARGUMENT;
  const size_t tok = (size_t)(B * H * N * D) * esize_of(dtype);
  const size_t lat = (size_t)(H * M * D) * esize_of(dtype);
  if (overlaps(y, tok, k, tok) || overlaps(y, tok, v, tok) || overlaps(y, tok, q, lat))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  if ((st = check_workspace(p, ws, ws_bytes)) != FLAREPP_OK) return st;
  Saved sv = saved_layout(B, H, N, M, D, saved);
  if (saved && (saved_bytes < sv.floats * sizeof(float) ||
                (reinterpret_cast<uintptr_t>(saved) & 15)))
    return FLAREPP_ERR_WORKSPACE;
  if (outputs_alias({{y, tok}, {saved, saved ? sv.floats * 4 : 0}, {ws, ws_bytes}},
                    {{q, lat}, {k, tok}, {v, tok}}))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  if ((st = check_device()) != FLAREPP_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const float c = (float)((double)scale * 1.4426950408889634);
  // the latents are scaled as the encoder and the decoder load them
  FLAREPP_TRY(launch_encode(dtype, (int)D,
                            encode_params(p, ws, q, 0, M * D, k, v, nullptr, c), s));
  FLAREPP_TRY(value_operand(p, ws, p.nchunks, nullptr, saved ? sv.z : nullptr, s,
                            saved ? sv.lse1 : nullptr));
  FLAREPP_TRY(decode(p, ws, q, 0, M * D, k, y, s, saved ? sv.lse2 : nullptr, c));
  return FLAREPP_OK;
}


}  // namespace

extern "C" {

const char* flarepp_status_string(int status) {
  switch (status) {
    case FLAREPP_OK: return "FLAREPP_OK";
    case FLAREPP_ERR_INVALID_ARGUMENT: return "FLAREPP_ERR_INVALID_ARGUMENT";
    case FLAREPP_ERR_UNSUPPORTED: return "FLAREPP_ERR_UNSUPPORTED";
    case FLAREPP_ERR_WORKSPACE: return "FLAREPP_ERR_WORKSPACE";
    case FLAREPP_ERR_HIP: return "FLAREPP_ERR_HIP";
    default: return "FLAREPP_UNKNOWN_STATUS";
  }
}

const char* flarepp_version(void) { return "0.1.0"; }

size_t flarepp_workspace_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype) {
  Plan p;
  if (make_plan(B, H, N, M, D, dtype, 0, &p) != FLAREPP_OK) return 0;
  return p.total;
}

size_t flare_encode_workspace_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                   int dtype, int64_t chunk_tokens) {
  Plan p;
  if (make_plan(B, H, N, M, D, dtype, chunk_tokens, &p) != FLAREPP_OK) return 0;
  return p.total;
}

size_t flare_decode_workspace_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                   int dtype) {
  return flarepp_workspace_size(B, H, N, M, D, dtype);
}

int flarepp_mixer_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                      const void* q0, const void* q_fixed, const float* gate, const void* k0,
                      const void* k, const void* v, void* y, void* workspace,
                      size_t workspace_bytes, void* stream) {
  try {
    if (!q_fixed || !gate) return FLAREPP_ERR_INVALID_ARGUMENT;
    return mixer_impl(B, H, N, M, D, dtype, q0, q_fixed, gate, k0, k0, k, v, y, workspace,
                      workspace_bytes, stream, nullptr);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int simplified_flarepp_mixer_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 int dtype, const void* q0, const void* k0, const void* v0,
                                 const void* k, const void* v, void* y, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  try {
    return mixer_impl(B, H, N, M, D, dtype, q0, nullptr, nullptr, k0, v0, k, v, y, workspace,
                      workspace_bytes, stream, nullptr);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int flarepp_mixer_fwd_noalloc(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                              int dtype, const void* q0, const void* q_fixed, const float* gate,
                              const void* k0, const void* k, const void* v, void* y,
                              void* stream) {
  try {
    if (!q_fixed || !gate) return FLAREPP_ERR_INVALID_ARGUMENT;
    return mixer_impl(B, H, N, M, D, dtype, q0, q_fixed, gate, k0, k0, k, v, y, nullptr,
                      (size_t)FLAREPP_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, 0, true);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int flarepp_mixer_fwd_timed(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                            const void* q0, const void* q_fixed, const float* gate,
                            const void* k0, const void* k, const void* v, void* y,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events) {
  try {
    if (events == nullptr) return FLAREPP_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < FLAREPP_TIMED_EVENTS; ++i)
      if (events[i] == nullptr) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (!q_fixed || !gate) return FLAREPP_ERR_INVALID_ARGUMENT;
    return mixer_impl(B, H, N, M, D, dtype, q0, q_fixed, gate, k0, k0, k, v, y, workspace,
                      workspace_bytes, stream, events);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int flare_mixer_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                    float scale, const void* q, const void* k, const void* v, void* y,
                    void* workspace, size_t workspace_bytes, void* stream) {
  try {
    return flare_impl(B, H, N, M, D, dtype, scale, q, k, v, y, workspace, workspace_bytes,
                      stream);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int flare_encode_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                     float scale, const void* q, int64_t q_batch_stride, const void* k,
                     const void* v, float* z, int64_t chunk_tokens, void* workspace,
                     size_t workspace_bytes, void* stream) {
  try {
    if (!q || !k || !v || !z) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(z))
      return FLAREPP_ERR_INVALID_ARGUMENT;
    Plan p;
    int st = make_plan(B, H, N, M, D, dtype, chunk_tokens, &p);
    if (st != FLAREPP_OK) return st;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (q_batch_stride != 0 && q_batch_stride != H * M * D) return FLAREPP_ERR_INVALID_ARGUMENT;
    const size_t tok = (size_t)(B * H * N * D) * esize_of(dtype);
    const size_t zb = (size_t)(B * H * M * D) * 4;
    const size_t lat = (size_t)((q_batch_stride ? B : 1) * H * M * D) * esize_of(dtype);
    if (overlaps(z, zb, k, tok) || overlaps(z, zb, v, tok) || overlaps(z, zb, q, lat))
      return FLAREPP_ERR_INVALID_ARGUMENT;
    if ((st = check_workspace(p, workspace, workspace_bytes)) != FLAREPP_OK) return st;
    if (outputs_alias({{z, zb}, {workspace, workspace_bytes}}, {{q, lat}, {k, tok}, {v, tok}}))
      return FLAREPP_ERR_INVALID_ARGUMENT;
    if ((st = check_device()) != FLAREPP_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float c = (float)((double)scale * 1.4426950408889634);
    FLAREPP_TRY(launch_encode(dtype, (int)D,
                              encode_params(p, workspace, q, q_batch_stride, M * D, k, v,
                                            nullptr, c),
                              s));
    FLAREPP_TRY(value_operand(p, workspace, p.nchunks, nullptr, z, s));
    return FLAREPP_OK;
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int flare_decode_fwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                     float scale, const void* q, int64_t q_batch_stride, const float* z,
                     const void* k, void* y, void* workspace, size_t workspace_bytes,
                     void* stream) {
  try {
    if (!q || !z || !k || !y) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(z) || !aligned16(k) || !aligned16(y))
      return FLAREPP_ERR_INVALID_ARGUMENT;
    Plan p;
    int st = make_plan(B, H, N, M, D, dtype, 0, &p);
    if (st != FLAREPP_OK) return st;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (q_batch_stride != 0 && q_batch_stride != H * M * D) return FLAREPP_ERR_INVALID_ARGUMENT;
    const size_t tok = (size_t)(B * H * N * D) * esize_of(dtype);
    const size_t zb = (size_t)(B * H * M * D) * 4;
    const size_t lat = (size_t)((q_batch_stride ? B : 1) * H * M * D) * esize_of(dtype);
    if (overlaps(y, tok, k, tok) || overlaps(y, tok, z, zb) || overlaps(y, tok, q, lat))
      return FLAREPP_ERR_INVALID_ARGUMENT;
    if ((st = check_workspace(p, workspace, workspace_bytes)) != FLAREPP_OK) return st;
    if (outputs_alias({{y, tok}, {workspace, workspace_bytes}}, {{q, lat}, {z, zb}, {k, tok}}))
      return FLAREPP_ERR_INVALID_ARGUMENT;
    if ((st = check_device()) != FLAREPP_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float c = (float)((double)scale * 1.4426950408889634);
    FLAREPP_TRY(value_operand(p, workspace, 0, z, nullptr, s));
    FLAREPP_TRY(decode(p, workspace, q, q_batch_stride, M * D, k, y, s, nullptr, c));
    return FLAREPP_OK;
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}


size_t flarepp_saved_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D) {
  if (check_shape(B, H, N, M, D, FLAREPP_BF16) == FLAREPP_ERR_INVALID_ARGUMENT) return 0;
  return saved_layout(B, H, N, M, D, nullptr).floats * sizeof(float);
}

int flarepp_mixer_fwd_train(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                            const void* q0, const void* q_fixed, const float* gate,
                            const void* k0, const void* k, const void* v, void* y, float* saved,
                            size_t saved_bytes, void* workspace, size_t workspace_bytes,
                            void* stream) {
  try {
    if (!q_fixed || !gate || !saved) return FLAREPP_ERR_INVALID_ARGUMENT;
    return mixer_impl(B, H, N, M, D, dtype, q0, q_fixed, gate, k0, k0, k, v, y, workspace,
                      workspace_bytes, stream, nullptr, saved, saved_bytes);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int flare_mixer_fwd_train(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                          float scale, const void* q, const void* k, const void* v, void* y,
                          float* saved, size_t saved_bytes, void* workspace,
                          size_t workspace_bytes, void* stream) {
  try {
    if (!saved) return FLAREPP_ERR_INVALID_ARGUMENT;
    return flare_impl(B, H, N, M, D, dtype, scale, q, k, v, y, workspace, workspace_bytes,
                      stream, saved, saved_bytes);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int simplified_flarepp_mixer_fwd_train(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                       int dtype, const void* q0, const void* k0, const void* v0,
                                       const void* k, const void* v, void* y, float* saved,
                                       size_t saved_bytes, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  try {
    if (!saved) return FLAREPP_ERR_INVALID_ARGUMENT;
    return mixer_impl(B, H, N, M, D, dtype, q0, nullptr, nullptr, k0, v0, k, v, y, workspace,
                      workspace_bytes, stream, nullptr, saved, saved_bytes);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

}  // extern "C"
