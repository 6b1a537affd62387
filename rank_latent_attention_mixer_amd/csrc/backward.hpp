// Parameters and launchers of the backward kernels (backward.hip).
#pragma once

#include "kernels.hpp"

namespace flarepp {

// ---------------------------------------------------------------------------
// Backward pass (bf16 / fp16, D in {16, 32, 64}).  All gradients are fp32.
//
// Every probability is recomputed as 2^(S' + C) with S' = c k.q from the
// score product and C (the product's accumulator input) holding minus the
// saved base-2 log-sum-exp of its softmax row, so P is the normalised
// attention weight; the Delta terms of the softmax Jacobian enter the second
// product the same way.  Weights normalised over the N tokens carry an extra
// factor 2^shift, and the latent-side gradient operands (dz', dqd') are
// divided by a power of two per (b, h) that brings their largest element to
// (1/2, 1]; both are undone in fp32 (the per-set exponent e = log2 rho -
// shift), so fp16 operands stay normal numbers.
// ---------------------------------------------------------------------------
enum { kBwdLatDec = 0, kBwdLatEnc = 1, kBwdLatSyn = 2 };
enum { kBwdTokFlare = 0, kBwdTokSyn = 1 };

// Latents in registers, tokens streamed: per-chunk sums over tokens,
// written to part[0] (Y = sum_n T_nm t0_n) and, for the decoder, part[1]
// (X = sum_n P_nm t1_n).
//   Dec: P = A2 (C = -lse2 per token), G = dy.z - Delta2 (C per token)
//   Enc: P = A1 2^shift (C = shift - lse1 per latent), G = v.dz' - Delta1'
//   Syn: as Enc over the synthesis (score and G token rows both k0)
// (Y of Enc/Syn carries the factor 2^-e of its set.)
struct BwdLatParams {
  const void* qop;              // score operand rows (scaled by c), dtype [.., Mpad, D]
  int64_t q_b_stride, q_h_stride;
  const void* gop;              // G operand rows, dtype [sets][Mpad][D]
  const float* lse;             // Enc/Syn: per-latent lse [sets][M]
  const float* negg;            // Enc/Syn: per-latent C of G [sets][M]
  const float* tok_lse;         // Dec: per-token lse2 [sets][N]
  const float* tok_negd;        // Dec: per-token -Delta2 [sets][N] (read unless formed here)
  const void* y_tok;            // Dec, where the pass forms -Delta2: y [B,H,N,D] dtype
  float* negd_out;              // ... and where it stores it [sets][N]
  float* lse_min_out;           // Dec, optional: partial minima of lse2 [sets][nchunks][2]
  const void* t[2];             // token tensors [B,H,N,D] dtype: score rows / Y, G rows / X
  float* part[2];               // [sets][nchunks][Mpad][D]: Y, X
  int B, H;
  int64_t N;
  int M, Mpad;
  int64_t chunk_tokens;
  int nchunks;
  const float* gate;            // non-null: skip heads with sigma == 0
  float shift;
};

// Tokens in registers, all latents resident in LDS: per-token results.
//   P1 = A 2^shift (per-latent C), P2 = A2 2^-e (flare, per-token C),
//   T = P1 G2 (+ P2 G1), Y = sum_m T_mn lat0_m, X = sum_m P1_mn lat2_m;
//   out0 = 2^e (s/c) Y and out1 = 2^e X, or, with out1 null,
//   out0 = 2^e (X + (s/c) Y) (synthesis with values = keys).
struct BwdTokParams {
  const void* lat[3];           // latent rows dtype: score/Y, G1 (flare), G2/X
  int64_t lat_b_stride[3], lat_h_stride[3];
  const float* lat_lse;         // per-latent lse of P1 [sets][lat_stat_stride]
  const float* lat_negd;        // per-latent C of G2 [sets][lat_stat_stride]
  int64_t lat_stat_stride;      // set stride of lat_lse / lat_negd (0: M)
  const void* kt;               // token score operand [B,H,N,D]
  const void* g1t;              // flare: token operand of G1 (dy)
  const void* g2t;              // token operand of G2 (v; synthesis: its values)
  const float* tok_lse;         // flare: per-token lse2 [sets][N]
  const float* tok_negd;        // flare: per-token -Delta2 [sets][N]
  float* out0;                  // [B,H,N,D] fp32
  float* out1;                  // [B,H,N,D] fp32 or null
  const float* set_e;           // [sets]: e of the latent operand's normaliser
  float s_over_c, shift;
  const float* gate;
  int B, H;
  int64_t N;
  int M;                        // latents this launch covers
  int wg_per_bh;
  int accumulate;               // add into out0/out1 instead of storing
  const float* tok_lse_min;     // flare: [sets][lse_min_parts] partial minima of tok_lse
  int lse_min_parts;
};

// -Delta2 = -(dy . y) per token row.
struct BwdPrepParams {
  const void *dy, *y;           // [rows][D] dtype
  float* negd;                  // [rows]
  int64_t rows;
  int D, dtype;
};

struct BwdRowsParams {
  const void* in;
  int in_dtype, in_sets;
  int64_t in_set_stride;
  void* out;                    // dtype [sets][Mpad][D]
  int dtype, sets, M, Mpad, D;
  float scale;
};

// After the decoder's latent pass: dq = s Y, dz = X (chunk sums).
struct BwdSumsParams {
  const float* part[2];         // Y, X
  int nchunks, Mpad, M, D, sets;
  float* dq;                    // [sets][M][D]
  float* dz;                    // [sets][M][D]
  float s;
};

// dst (+)= s 2^e[set] * sum over chunks of Y.
struct BwdAddParams {
  const float* part;            // [sets][nchunks][Mpad][D]
  int nchunks, Mpad, M, D, sets;
  float* dst;                   // [sets][M][D]
  const float* set_e;           // [sets] or null (e = 0)
  float s;
  int accumulate;
};

// One workgroup per set: g = alpha src (alpha = sigma(gate[h]), or 1),
// rho = 2^ceil(log2 max|g|);  rows = g / rho, negd = -(g . w) / rho per
// latent, e = log2 rho - shift.
struct BwdNormParams {
  const float* src;             // [sets][M][D]
  const float* w;               // [sets][M][D]
  const float* gate;            // [H] or null
  void* rows;                   // dtype [sets][Mpad][D]
  float* negd;                  // [sets][M]
  float* set_e;                 // [sets]
  int H, M, Mpad, D, sets, dtype;
  float shift;
};

struct BwdGateParams {
  int H, B, M, Mpad, D;
  const float* gate;            // null: sigma = 1
  const float* dq;              // [sets][M][D]
  const float* qd;              // [sets][M][D] (saved q_dyn)
  float* dqf;                   // [H][M][D]  sum over the batch
  float* dgate;                 // [H] or null
  int synthesis;                // 0: only dqf
};

hipError_t launch_bwd_lat(int dtype, int mode, int D, const BwdLatParams& p, hipStream_t s);
hipError_t launch_bwd_tok(int dtype, int mode, int D, const BwdTokParams& p, hipStream_t s);
hipError_t launch_bwd_tok_prep(const BwdPrepParams& p, hipStream_t s);
hipError_t launch_bwd_rows(const BwdRowsParams& p, hipStream_t s);
hipError_t launch_bwd_dec_sums(const BwdSumsParams& p, hipStream_t s);
hipError_t launch_bwd_add_sums(const BwdAddParams& p, hipStream_t s);
hipError_t launch_bwd_gate(const BwdGateParams& p, hipStream_t s);
hipError_t launch_bwd_norm(const BwdNormParams& p, hipStream_t s);
int bwd_latents_per_block(int D);
// Whether the decoder's latent pass forms -Delta2 itself (then no separate
// per-token pass runs before it).
bool bwd_lat_forms_delta2(int D);
int bwd_tokens_per_tile();
size_t bwd_tok_lds_bytes(int M, int D);
// Dynamic LDS one token-pass workgroup may hold (the CU's 160 KB, less
// room for the kernel's small static reduction buffer).
constexpr size_t kBwdTokMaxLds = 160 * 1024 - 512;
// Launches over latent ranges the token pass takes for M latents (0: none fits).
int bwd_tok_latent_ranges(int M, int D);

// ---------------------------------------------------------------------------
// VALU backward (backward_valu.hip): fp32 at every D, bf16 / fp16 at D = 8.
// One thread per latent row (latent pass) or per token (token pass), fp32
// arithmetic; weights A = 2^(S' - lse) from the saved normalisers, S' from
// c q rounded to `round_dtype` as the forward's operand was.
// ---------------------------------------------------------------------------
struct BwdValuLatParams {
  int mode;                     // kBwdLatDec / kBwdLatEnc / kBwdLatSyn
  const void* qlat;             // latent rows (unscaled) [.., M, D] in qlat_dtype
  int qlat_dtype;
  int64_t q_b_stride, q_h_stride;
  float c;                      // score factor s log2(e)
  int round_dtype;              // dtype c q is rounded to (kF32: none)
  const float* glat;            // fp32 [sets][M][D]: Dec z, Enc dz, Syn dqd
  const float* lse_lat;         // Enc/Syn: [sets][M]
  const float* negd_lat;        // Enc/Syn: -Delta per latent [sets][M]
  const float* lse_tok;         // Dec: lse2 [sets][N]
  const float* negd_tok;        // Dec: -Delta2 [sets][N]
  const void* tk;               // token score rows [B,H,N,D] (k or k0)
  const void* tg;               // token rows of G: Dec dy, Enc v, Syn values
  float* part_y;                // [sets][nchunks][M][D]: s sum A G k
  float* part_x;                // Dec: [sets][nchunks][M][D]: sum A dy
  int B, H;
  int64_t N;
  int M;
  int64_t chunk_tokens;
  int nchunks;
  float s;
  const float* gate;            // Syn: heads with sigma == 0 write zeros
};

struct BwdValuTokParams {
  int mode;                     // kBwdTokFlare / kBwdTokSyn
  const void* qlat;
  int qlat_dtype;
  int64_t q_b_stride, q_h_stride;
  float c;
  int round_dtype;
  const float* lat_z;           // Flare: z [sets][M][D]
  const float* lat_g;           // Flare: dz; Syn: dqd [sets][M][D]
  const float* lse_lat;         // Flare: lse1; Syn: lse0 [sets][M]
  const float* negd_lat;        // Flare: -Delta1; Syn: -Delta0 [sets][M]
  const float* lse_tok;         // Flare: lse2 [sets][N]
  const float* negd_tok;        // Flare: -Delta2 [sets][N]
  const void* tk;               // token score rows (k or k0)
  const void* tdy;              // Flare: dy
  const void* tw;               // Flare: v; Syn: the synthesis values (k0 or v0)
  float* out_k;                 // dk (Syn: dk0, plus the value part when out_v is null)
  float* out_v;                 // dv (Syn: dv0) or null
  int B, H;
  int64_t N;
  int M;
  float s_over_c;
  const float* gate;
};

hipError_t launch_bwd_valu_lat(int dtype, int D, const BwdValuLatParams& p, hipStream_t s);
hipError_t launch_bwd_valu_tok(int dtype, int D, const BwdValuTokParams& p, hipStream_t s);
hipError_t launch_bwd_valu_negd(int dtype, int D, const void* dy, const void* y, float* out,
                                int64_t rows, hipStream_t s);
hipError_t launch_bwd_valu_sum(int D, const float* part, int nchunks, int M, int sets, float* dst,
                               int accumulate, const float* w, float* negd, hipStream_t s);
hipError_t launch_bwd_valu_batch_sum(const float* src, int B, int H, int M, int D, float* out,
                                     const float* gate, float* dqd, hipStream_t s);
hipError_t launch_bwd_valu_negd_rows(const float* a, const float* w, int64_t rows, int D,
                                     float* out, hipStream_t s);
hipError_t launch_bwd_valu_gate(const float* dq, const float* qd, int B, int H, int M, int D,
                                const float* gate, float* dgate, hipStream_t s);

}  // namespace flarepp
