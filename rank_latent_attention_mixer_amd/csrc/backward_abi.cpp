// C boundary of the backward pass: argument validation, workspace carving
// and the launch sequence of the training entry points (include/flarepp.h).
// The gradients follow from the forward of the FLARE.py README ("FLARE++"
// and "FLARE" listings) by the chain rule.
#include <cmath>
#include <cstring>

#include "abi_common.hpp"
#include "backward.hpp"

namespace {

using namespace flarepp;

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------

constexpr int kBwdTargetWgs = 512;

struct BwdPlan {
  int64_t B, H, N, M, D;
  int dtype, Mpad, nchunks, mblocks, tok_wg_per_bh;
  int64_t chunk_tokens;
  size_t off_cq, off_zr, off_nd2, off_py, off_px, off_dq, off_dz, off_dzp, off_nd1, off_e1,
      off_cq0, off_dqdp, off_nd0, off_e0, off_dq0s, off_l2min, total;
};

// fp32 at every D, and D = 8 in any dtype, run on the VALU kernels
// (backward_valu.hip); the rest on the matrix cores.
bool bwd_on_valu(int dtype, int64_t D) { return dtype == FLAREPP_F32 || D < 16; }

struct ValuPlan {
  int64_t chunk_tokens;
  int nchunks;
  size_t off_nd2, off_py, off_px, off_dq, off_dz, off_nd1, off_dqd, off_nd0, off_dq0s, total;
};

int make_valu_plan(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, ValuPlan* p) {
  const int64_t BH = B * H;
  // token chunks of the latent passes: about 2048 workgroups of 64 latents
  const int64_t mblocks = (M + 63) / 64;
  int64_t c = (2048 + BH * mblocks - 1) / (BH * mblocks);
  const int64_t tiles = (N + 31) / 32;
  if (c > tiles) c = tiles;
  if (c < 1) c = 1;
  p->chunk_tokens = (tiles + c - 1) / c * 32;
  p->nchunks = (int)((N + p->chunk_tokens - 1) / p->chunk_tokens);
  int64_t wgs;
  if (!mul_ok(BH * mblocks, p->nchunks, &wgs) || wgs > 0x7FFFFFFF || BH > 65535)
    return FLAREPP_ERR_INVALID_ARGUMENT;
  const size_t f = 4, rows = (size_t)BH * M * D;
  const size_t part = (size_t)BH * p->nchunks * M * D * f;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  p->off_nd2 = take((size_t)BH * N * f);
  p->off_py = take(part);
  p->off_px = take(part);
  p->off_dq = take(rows * f);
  p->off_dz = take(rows * f);
  p->off_nd1 = take((size_t)BH * M * f);
  p->off_dqd = take(rows * f);
  p->off_nd0 = take((size_t)BH * M * f);
  p->off_dq0s = take(rows * f);
  p->total = off;
  return FLAREPP_OK;
}

int make_bwd_plan(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, BwdPlan* p) {
  int st = check_shape(B, H, N, M, D, dtype);
  if (st != FLAREPP_OK) return st;
  if (bwd_on_valu(dtype, D)) {
    ValuPlan vp;
    if ((st = make_valu_plan(B, H, N, M, D, &vp)) != FLAREPP_OK) return st;
    std::memset(p, 0, sizeof(*p));
    p->B = B; p->H = H; p->N = N; p->M = M; p->D = D; p->dtype = dtype;
    p->total = vp.total;
    return FLAREPP_OK;
  }
  if (bwd_tok_latent_ranges((int)M, (int)D) < 1) return FLAREPP_ERR_UNSUPPORTED;
  p->B = B; p->H = H; p->N = N; p->M = M; p->D = D; p->dtype = dtype;
  p->Mpad = (int)((M + 31) / 32 * 32);
  const int64_t BH = B * H;
  p->mblocks = (int)((M + bwd_latents_per_block((int)D) - 1) / bwd_latents_per_block((int)D));
  const int64_t unit = 128;
  const int64_t tiles = (N + unit - 1) / unit;
  int64_t c = (kBwdTargetWgs + BH * p->mblocks - 1) / (BH * p->mblocks);
  if (c < 1) c = 1;
  if (c > tiles) c = tiles;
  p->chunk_tokens = (tiles + c - 1) / c * unit;
  p->nchunks = (int)((N + p->chunk_tokens - 1) / p->chunk_tokens);
  int64_t w = (kDecTargetWgs + BH - 1) / BH;
  const int64_t ttiles = (N + bwd_tokens_per_tile() - 1) / bwd_tokens_per_tile();
  if (w > ttiles) w = ttiles;
  if (w < 1) w = 1;
  p->tok_wg_per_bh = (int)w;
  int64_t wgs;
  if (!mul_ok(BH * p->mblocks, p->nchunks, &wgs) || wgs > 0x7FFFFFFF) return FLAREPP_ERR_INVALID_ARGUMENT;
  const size_t es = 2, f = 4;
  const size_t rows = (size_t)BH * p->Mpad * D;
  const size_t part = (size_t)BH * p->nchunks * p->Mpad * D * f;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  p->off_cq = take(rows * es);
  p->off_zr = take(rows * es);
  p->off_nd2 = take((size_t)BH * N * f);
  p->off_py = take(part);
  p->off_px = take(part);
  p->off_dq = take((size_t)BH * M * D * f);
  p->off_dz = take((size_t)BH * M * D * f);
  p->off_dzp = take(rows * es);
  p->off_nd1 = take((size_t)BH * M * f);
  p->off_e1 = take((size_t)BH * f);
  p->off_cq0 = take((size_t)H * p->Mpad * D * es);
  p->off_dqdp = take(rows * es);
  p->off_nd0 = take((size_t)BH * M * f);
  p->off_e0 = take((size_t)BH * f);
  p->off_dq0s = take((size_t)BH * M * D * f);
  p->off_l2min = take((size_t)BH * p->nchunks * 2 * f);
  p->total = off;
  return FLAREPP_OK;
}

// The VALU sequence (fp32, or D = 8): the same passes as the matrix-core
// sequence below, one thread per latent row or token.
int bwd_valu_run(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, float scale,
                 float c, bool pp, bool simplified, const void* q0, const float* gate,
                 const void* k0, const void* v0, const void* q_flare, const void* k,
                 const void* v, const void* y, const void* dy, const Saved& sv, float* dq0,
                 float* dq_lat, float* dgate, float* dk0, float* dv0, float* dk, float* dv,
                 void* ws, hipStream_t s) {
  ValuPlan p;
  int st = make_valu_plan(B, H, N, M, D, &p);
  if (st != FLAREPP_OK) return st;
  const int64_t BH = B * H;
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(ws_at(ws, off)); };
  // -Delta2 = -(dy . y) per token
  FLAREPP_TRY(launch_bwd_valu_negd(dtype, (int)D, dy, y, f32(p.off_nd2), BH * N, s));
  // decoder over tokens: dq = s dS2^T k, dz = A2^T dy
  BwdValuLatParams lp;
  std::memset(&lp, 0, sizeof(lp));
  lp.mode = kBwdLatDec;
  if (pp) {
    lp.qlat = sv.q; lp.qlat_dtype = FLAREPP_F32; lp.q_b_stride = H * M * D; lp.q_h_stride = M * D;
  } else {
    lp.qlat = q_flare; lp.qlat_dtype = dtype; lp.q_b_stride = 0; lp.q_h_stride = M * D;
  }
  lp.c = c; lp.round_dtype = dtype;
  lp.glat = sv.z; lp.lse_tok = sv.lse2; lp.negd_tok = f32(p.off_nd2);
  lp.tk = k; lp.tg = dy; lp.part_y = f32(p.off_py); lp.part_x = f32(p.off_px);
  lp.B = (int)B; lp.H = (int)H; lp.N = N; lp.M = (int)M;
  lp.chunk_tokens = p.chunk_tokens; lp.nchunks = p.nchunks; lp.s = scale;
  FLAREPP_TRY(launch_bwd_valu_lat(dtype, (int)D, lp, s));
  FLAREPP_TRY(launch_bwd_valu_sum((int)D, f32(p.off_py), p.nchunks, (int)M, (int)BH, f32(p.off_dq),
                                  0, nullptr, nullptr, s));
  // dz, and -Delta1 = -(dz . z) per latent
  FLAREPP_TRY(launch_bwd_valu_sum((int)D, f32(p.off_px), p.nchunks, (int)M, (int)BH, f32(p.off_dz),
                                  0, sv.z, f32(p.off_nd1), s));
  // encoder over tokens: dq += s dS1 k
  lp.mode = kBwdLatEnc;
  lp.glat = f32(p.off_dz); lp.lse_lat = sv.lse1; lp.negd_lat = f32(p.off_nd1);
  lp.lse_tok = nullptr; lp.negd_tok = nullptr; lp.tg = v; lp.part_x = nullptr;
  FLAREPP_TRY(launch_bwd_valu_lat(dtype, (int)D, lp, s));
  FLAREPP_TRY(launch_bwd_valu_sum((int)D, f32(p.off_py), p.nchunks, (int)M, (int)BH, f32(p.off_dq),
                                  1, nullptr, nullptr, s));
  // per token, both attentions: dk = s (dS2 + dS1^T) q, dv = A1^T dz
  BwdValuTokParams kp;
  std::memset(&kp, 0, sizeof(kp));
  kp.mode = kBwdTokFlare;
  kp.qlat = lp.qlat; kp.qlat_dtype = lp.qlat_dtype;
  kp.q_b_stride = lp.q_b_stride; kp.q_h_stride = lp.q_h_stride;
  kp.c = c; kp.round_dtype = dtype;
  kp.lat_z = sv.z; kp.lat_g = f32(p.off_dz); kp.lse_lat = sv.lse1; kp.negd_lat = f32(p.off_nd1);
  kp.lse_tok = sv.lse2; kp.negd_tok = f32(p.off_nd2);
  kp.tk = k; kp.tdy = dy; kp.tw = v; kp.out_k = dk; kp.out_v = dv;
  kp.B = (int)B; kp.H = (int)H; kp.N = N; kp.M = (int)M; kp.s_over_c = scale / c;
  FLAREPP_TRY(launch_bwd_valu_tok(dtype, (int)D, kp, s));
  if (!pp) {  // FLARE: the latents are shared by the batch
    FLAREPP_TRY(launch_bwd_valu_batch_sum(f32(p.off_dq), (int)B, (int)H, (int)M, (int)D, dq_lat,
                                          nullptr, nullptr, s));
    return FLAREPP_OK;
  }
  // FLARE++: dq_fixed = sum_b dq, dqd = sigma dq, dgate; simplified: dqd = dq
  FLAREPP_TRY(launch_bwd_valu_batch_sum(f32(p.off_dq), (int)B, (int)H, (int)M, (int)D,
                                        simplified ? nullptr : dq_lat,
                                        simplified ? nullptr : gate, f32(p.off_dqd), s));
  if (!simplified)
    FLAREPP_TRY(launch_bwd_valu_gate(f32(p.off_dq), sv.qd, (int)B, (int)H, (int)M, (int)D, gate,
                                     dgate, s));
  // -Delta0 = -(dqd . q_dyn) per latent
  FLAREPP_TRY(launch_bwd_valu_negd_rows(f32(p.off_dqd), sv.qd, BH * M, (int)D, f32(p.off_nd0), s));
  // synthesis over tokens: dq0 = s dS0 k0 per (b, h), then summed over the batch
  lp.mode = kBwdLatSyn;
  lp.qlat = q0; lp.qlat_dtype = dtype; lp.q_b_stride = 0; lp.q_h_stride = M * D;
  lp.glat = f32(p.off_dqd); lp.lse_lat = sv.lse0; lp.negd_lat = f32(p.off_nd0);
  lp.tk = k0; lp.tg = v0; lp.gate = gate;
  FLAREPP_TRY(launch_bwd_valu_lat(dtype, (int)D, lp, s));
  FLAREPP_TRY(launch_bwd_valu_sum((int)D, f32(p.off_py), p.nchunks, (int)M, (int)BH,
                                  f32(p.off_dq0s), 0, nullptr, nullptr, s));
  FLAREPP_TRY(launch_bwd_valu_batch_sum(f32(p.off_dq0s), (int)B, (int)H, (int)M, (int)D, dq0,
                                        nullptr, nullptr, s));
  // dk0 = s dS0^T q0 (+ A0^T dqd when k0 is also the value), dv0 = A0^T dqd
  kp.mode = kBwdTokSyn;
  kp.qlat = q0; kp.qlat_dtype = dtype; kp.q_b_stride = 0; kp.q_h_stride = M * D;
  kp.lat_z = nullptr; kp.lat_g = f32(p.off_dqd); kp.lse_lat = sv.lse0;
  kp.negd_lat = f32(p.off_nd0); kp.lse_tok = nullptr; kp.negd_tok = nullptr;
  kp.tk = k0; kp.tdy = nullptr; kp.tw = v0;
  kp.out_k = dk0; kp.out_v = simplified ? dv0 : nullptr; kp.gate = gate;
  FLAREPP_TRY(launch_bwd_valu_tok(dtype, (int)D, kp, s));
  return FLAREPP_OK;
}

// Shared by FLARE++ (q0 non-null, v0 == k0: synthesis and gate), the
// simplified mixer (q0 non-null, v0 its own tensor, no gate: q = q_dyn) and
// FLARE (q0 null, q given, caller scale).
int bwd_impl(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype, float scale,
             const void* q0, const float* gate, const void* k0, const void* v0,
             const void* q_flare, const void* k, const void* v, const void* y, const void* dy,
             const float* saved, size_t saved_bytes, float* dq0, float* dq_lat, float* dgate,
             float* dk0, float* dv0, float* dk, float* dv, void* ws, size_t ws_bytes,
             void* stream) {
  const bool pp = q0 != nullptr;
  const bool simplified = pp && v0 != k0;
  if (!k || !v || !y || !dy || !saved || !dk || !dv) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (pp && (!k0 || !v0 || !dq0 || !dk0)) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (pp && !simplified && (!gate || !dgate || !dq_lat)) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (simplified && !dv0) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (!pp && (!q_flare || !dq_lat)) return FLAREPP_ERR_INVALID_ARGUMENT;
  if (simplified) gate = nullptr;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FLAREPP_ERR_INVALID_ARGUMENT;
  BwdPlan p;
  int st = make_bwd_plan(B, H, N, M, D, dtype, &p);
  if (st != FLAREPP_OK) return st;
  Saved sv = saved_layout(B, H, N, M, D, const_cast<float*>(saved));
  if (saved_bytes < sv.floats * sizeof(float) || !aligned16(saved)) return FLAREPP_ERR_WORKSPACE;
  for (const void* g : {(const void*)dq_lat, (const void*)dk, (const void*)dv,
                        pp ? (const void*)dq0 : nullptr, pp ? (const void*)dk0 : nullptr,
                        simplified ? (const void*)dv0 : nullptr})
    if (g && !aligned16(g)) return FLAREPP_ERR_INVALID_ARGUMENT;
  for (const void* in : {k, v, y, dy, pp ? k0 : nullptr, pp ? v0 : nullptr})
    if (in && !aligned16(in)) return FLAREPP_ERR_INVALID_ARGUMENT;
  const size_t tokf = (size_t)(B * H * N * D) * 4, latf = (size_t)(H * M * D) * 4;
  const size_t es = (size_t)esize_of(dtype);
  const size_t toke = (size_t)(B * H * N * D) * es, late = (size_t)(H * M * D) * es;
  if (ws == nullptr || ws_bytes < p.total || ((uintptr_t)ws % kAlign) != 0)
    return FLAREPP_ERR_WORKSPACE;
  // the workspace is written by the kernels, so it counts as an output
  if (outputs_alias({{dq0, pp ? latf : 0}, {dq_lat, latf}, {dgate, dgate ? (size_t)H * 4 : 0},
                     {dk0, pp ? tokf : 0}, {dv0, simplified ? tokf : 0}, {dk, tokf}, {dv, tokf},
                     {ws, ws_bytes}},
                    {{q0, late}, {gate, gate ? (size_t)H * 4 : 0}, {k0, toke}, {v0, toke},
                     {q_flare, late}, {k, toke}, {v, toke}, {y, toke}, {dy, toke},
                     {saved, sv.floats * 4}}))
    return FLAREPP_ERR_INVALID_ARGUMENT;
  if ((st = check_device()) != FLAREPP_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  // the forward's score factor, bit for bit (it rounds c q to the operand type)
  const float c = pp ? (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634)
                     : (float)((double)scale * 1.4426950408889634);
  if (bwd_on_valu(dtype, D))
    return bwd_valu_run(B, H, N, M, D, dtype, scale, c, pp, simplified, q0, gate, k0, v0, q_flare,
                        k, v, y, dy, sv, dq0, dq_lat, dgate, dk0, dv0, dk, dv, ws, s);
  // weights normalised over the N tokens are taken times 2^shift so that
  // ~1/N stays a normal fp16 number while P times a gradient term stays
  // far below the fp16 maximum
  const float shift = (float)std::min(8.0, std::max(0.0, std::floor(std::log2((double)N)) - 8.0));
  const int64_t BH = B * H;
  const int64_t rowH = (int64_t)p.Mpad * D;   // elements per latent set of operand rows
  auto at = [&](size_t off) { return ws_at(ws, off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(ws_at(ws, off)); };

  // operand rows of the saved routing query (scaled) and z
  BwdRowsParams rp;
  rp.dtype = dtype; rp.M = (int)M; rp.Mpad = p.Mpad; rp.D = (int)D;
  if (pp) {
    rp.in = sv.q; rp.in_dtype = FLAREPP_F32; rp.in_sets = (int)BH; rp.in_set_stride = M * D;
  } else {
    rp.in = q_flare; rp.in_dtype = dtype; rp.in_sets = (int)H; rp.in_set_stride = M * D;
  }
  rp.sets = (int)BH; rp.out = at(p.off_cq); rp.scale = c;
  FLAREPP_TRY(launch_bwd_rows(rp, s));
  rp.in = sv.z; rp.in_dtype = FLAREPP_F32; rp.in_sets = (int)BH; rp.in_set_stride = M * D;
  rp.out = at(p.off_zr); rp.scale = 1.f;
  FLAREPP_TRY(launch_bwd_rows(rp, s));

  // -Delta2 per token: formed inside the decoder's latent pass where its
  // tile staging leaves threads free, else by a pass of its own
  const bool lat_delta = bwd_lat_forms_delta2((int)D);
  if (!lat_delta) {
    BwdPrepParams tp;
    tp.dy = dy; tp.y = y; tp.negd = f32(p.off_nd2);
    tp.rows = BH * N; tp.D = (int)D; tp.dtype = dtype;
    FLAREPP_TRY(launch_bwd_tok_prep(tp, s));
  }

  // decoder, sums over tokens: dz = A2^T dy, dq = s dS2^T k
  BwdLatParams lp;
  std::memset(&lp, 0, sizeof(lp));
  lp.qop = at(p.off_cq); lp.q_b_stride = H * rowH; lp.q_h_stride = rowH;
  lp.gop = at(p.off_zr);
  lp.tok_lse = sv.lse2; lp.tok_negd = f32(p.off_nd2);
  lp.y_tok = lat_delta ? y : nullptr; lp.negd_out = lat_delta ? f32(p.off_nd2) : nullptr;
  lp.lse_min_out = f32(p.off_l2min);
  lp.t[0] = k; lp.t[1] = dy;
  lp.part[0] = f32(p.off_py); lp.part[1] = f32(p.off_px);
  lp.B = (int)B; lp.H = (int)H; lp.N = N; lp.M = (int)M; lp.Mpad = p.Mpad;
  lp.chunk_tokens = p.chunk_tokens; lp.nchunks = p.nchunks; lp.shift = shift;
  FLAREPP_TRY(launch_bwd_lat(dtype, kBwdLatDec, (int)D, lp, s));
  BwdSumsParams sp;
  sp.part[0] = f32(p.off_py); sp.part[1] = f32(p.off_px);
  sp.nchunks = p.nchunks; sp.Mpad = p.Mpad; sp.M = (int)M; sp.D = (int)D; sp.sets = (int)BH;
  sp.dq = f32(p.off_dq); sp.dz = f32(p.off_dz); sp.s = scale;
  FLAREPP_TRY(launch_bwd_dec_sums(sp, s));
  // dz' rows and -Delta1 = -(dz . z), normalised per set
  BwdNormParams np;
  np.src = f32(p.off_dz); np.w = sv.z; np.gate = nullptr; np.rows = at(p.off_dzp);
  np.negd = f32(p.off_nd1); np.set_e = f32(p.off_e1);
  np.H = (int)H; np.M = (int)M; np.Mpad = p.Mpad; np.D = (int)D; np.sets = (int)BH;
  np.dtype = dtype; np.shift = shift;
  FLAREPP_TRY(launch_bwd_norm(np, s));
  // encoder, sums over tokens: dq += s dS1 k
  lp.gop = at(p.off_dzp);
  lp.lse = sv.lse1; lp.negg = f32(p.off_nd1);
  lp.tok_lse = nullptr; lp.tok_negd = nullptr; lp.y_tok = nullptr; lp.negd_out = nullptr;
  lp.lse_min_out = nullptr;
  lp.t[1] = v;
  FLAREPP_TRY(launch_bwd_lat(dtype, kBwdLatEnc, (int)D, lp, s));
  BwdAddParams ap;
  ap.part = f32(p.off_py); ap.nchunks = p.nchunks; ap.Mpad = p.Mpad; ap.M = (int)M;
  ap.D = (int)D; ap.sets = (int)BH; ap.dst = f32(p.off_dq); ap.s = scale; ap.accumulate = 1;
  ap.set_e = f32(p.off_e1);
  FLAREPP_TRY(launch_bwd_add_sums(ap, s));
  // per token, both attentions: dk = s (dS2 + dS1^T) q, dv = A1^T dz
  BwdTokParams kp;
  std::memset(&kp, 0, sizeof(kp));
  kp.lat[0] = at(p.off_cq); kp.lat[1] = at(p.off_zr); kp.lat[2] = at(p.off_dzp);
  for (int t = 0; t < 3; ++t) { kp.lat_b_stride[t] = H * rowH; kp.lat_h_stride[t] = rowH; }
  kp.lat_lse = sv.lse1; kp.lat_negd = f32(p.off_nd1);
  kp.kt = k; kp.g1t = dy; kp.g2t = v;
  kp.tok_lse = sv.lse2; kp.tok_negd = f32(p.off_nd2);
  kp.out0 = dk; kp.out1 = dv; kp.s_over_c = scale / c; kp.shift = shift;
  kp.set_e = f32(p.off_e1);
  kp.B = (int)B; kp.H = (int)H; kp.N = N; kp.M = (int)M; kp.wg_per_bh = p.tok_wg_per_bh;
  // partial minima of lse2 per set, from the decoder's latent pass: the
  // range test of the token pass's one-exponential form
  kp.tok_lse_min = f32(p.off_l2min); kp.lse_min_parts = 2 * p.nchunks;
  FLAREPP_TRY(launch_bwd_tok(dtype, kBwdTokFlare, (int)D, kp, s));

  // latent gradient summed over the batch; FLARE++: gate and synthesis operands
  BwdGateParams gp;
  std::memset(&gp, 0, sizeof(gp));
  gp.H = (int)H; gp.B = (int)B; gp.M = (int)M; gp.Mpad = p.Mpad; gp.D = (int)D;
  gp.gate = gate; gp.dq = f32(p.off_dq); gp.qd = sv.qd; gp.dqf = dq_lat; gp.dgate = dgate;
  gp.synthesis = pp && !simplified ? 1 : 0;
  if (!simplified) FLAREPP_TRY(launch_bwd_gate(gp, s));
  if (!pp) return FLAREPP_OK;

  // dqd' rows and -Delta0 = -(dqd . q_dyn), dqd = sigma dq (simplified:
  // sigma = 1), normalised per set
  np.src = f32(p.off_dq); np.w = sv.qd; np.gate = gate; np.rows = at(p.off_dqdp);
  np.negd = f32(p.off_nd0); np.set_e = f32(p.off_e0);
  FLAREPP_TRY(launch_bwd_norm(np, s));

  // synthesis: seeds as operand rows (shared over the batch)
  BwdRowsParams r0 = rp;
  r0.in = q0; r0.in_dtype = dtype; r0.in_sets = (int)H; r0.in_set_stride = M * D;
  r0.sets = (int)H; r0.out = at(p.off_cq0); r0.scale = c;
  FLAREPP_TRY(launch_bwd_rows(r0, s));
  // dq0 = s dS0 k0 per (b, h), then summed over the batch
  lp.qop = at(p.off_cq0); lp.q_b_stride = 0; lp.q_h_stride = rowH;
  lp.gop = at(p.off_dqdp); lp.lse = sv.lse0; lp.negg = f32(p.off_nd0);
  lp.t[0] = k0; lp.t[1] = simplified ? v0 : nullptr;
  lp.gate = gate;
  // with values k0 the G rows are the score rows (one token tensor)
  FLAREPP_TRY(launch_bwd_lat(dtype, simplified ? kBwdLatEnc : kBwdLatSyn, (int)D, lp, s));
  ap.dst = f32(p.off_dq0s); ap.accumulate = 0; ap.set_e = f32(p.off_e0);
  FLAREPP_TRY(launch_bwd_add_sums(ap, s));
  BwdGateParams g0 = gp;
  g0.dq = f32(p.off_dq0s); g0.dqf = dq0; g0.dgate = nullptr; g0.synthesis = 0;
  FLAREPP_TRY(launch_bwd_gate(g0, s));
  // dk0 = s dS0^T q0 and dv0 = A0^T dqd (FLARE++: k0 is key and value, the
  // two are summed)
  BwdTokParams k0p;
  std::memset(&k0p, 0, sizeof(k0p));
  k0p.lat[0] = at(p.off_cq0); k0p.lat_b_stride[0] = 0; k0p.lat_h_stride[0] = rowH;
  k0p.lat[2] = at(p.off_dqdp); k0p.lat_b_stride[2] = H * rowH; k0p.lat_h_stride[2] = rowH;
  k0p.lat_lse = sv.lse0; k0p.lat_negd = f32(p.off_nd0);
  k0p.kt = k0; k0p.g2t = v0;
  k0p.out0 = dk0; k0p.out1 = simplified ? dv0 : nullptr; k0p.s_over_c = scale / c; k0p.shift = shift;
  k0p.set_e = f32(p.off_e0);
  k0p.gate = gate;
  k0p.B = (int)B; k0p.H = (int)H; k0p.N = N; k0p.M = (int)M; k0p.wg_per_bh = p.tok_wg_per_bh;
  FLAREPP_TRY(launch_bwd_tok(dtype, kBwdTokSyn, (int)D, k0p, s));
  return FLAREPP_OK;
}

}  // namespace

extern "C" {

size_t flarepp_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                  int dtype) {
  BwdPlan p;
  if (make_bwd_plan(B, H, N, M, D, dtype, &p) != FLAREPP_OK) return 0;
  return p.total;
}

int flarepp_mixer_bwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                      const void* q0, const void* q_fixed, const float* gate, const void* k0,
                      const void* k, const void* v, const void* y, const void* dy,
                      const float* saved, size_t saved_bytes, float* dq0, float* dq_fixed,
                      float* dgate, float* dk0, float* dk, float* dv, void* workspace,
                      size_t workspace_bytes, void* stream) {
  try {
    if (!q0 || !q_fixed) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (!gate) return FLAREPP_ERR_INVALID_ARGUMENT;
    return bwd_impl(B, H, N, M, D, dtype, (float)(1.0 / std::sqrt((double)D)), q0, gate, k0,
                    k0, nullptr, k, v, y, dy, saved, saved_bytes, dq0, dq_fixed, dgate, dk0,
                    nullptr, dk, dv, workspace, workspace_bytes, stream);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int flare_mixer_bwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, int dtype,
                    float scale, const void* q, const void* k, const void* v, const void* y,
                    const void* dy, const float* saved, size_t saved_bytes, float* dq, float* dk,
                    float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!q) return FLAREPP_ERR_INVALID_ARGUMENT;
    return bwd_impl(B, H, N, M, D, dtype, scale, nullptr, nullptr, nullptr, nullptr, q, k, v, y,
                    dy, saved, saved_bytes, nullptr, dq, nullptr, nullptr, nullptr, dk, dv,
                    workspace, workspace_bytes, stream);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

int simplified_flarepp_mixer_bwd(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 int dtype, const void* q0, const void* k0, const void* v0,
                                 const void* k, const void* v, const void* y, const void* dy,
                                 const float* saved, size_t saved_bytes, float* dq0, float* dk0,
                                 float* dv0, float* dk, float* dv, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  try {
    if (!q0 || !k0 || !v0) return FLAREPP_ERR_INVALID_ARGUMENT;
    if (k0 == v0) return FLAREPP_ERR_INVALID_ARGUMENT;  // the FLARE++ entry point covers v0 == k0
    return bwd_impl(B, H, N, M, D, dtype, (float)(1.0 / std::sqrt((double)D)), q0, nullptr, k0,
                    v0, nullptr, k, v, y, dy, saved, saved_bytes, dq0, nullptr, nullptr, dk0,
                    dv0, dk, dv, workspace, workspace_bytes, stream);
  } catch (...) {
    return FLAREPP_ERR_HIP;
  }
}

}  // extern "C"
