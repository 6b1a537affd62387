// Host-side launch interface of the FLARE++ kernels.  Everything here is
// asynchronous on the given stream; shapes are validated by the caller
// (flarepp_abi.cpp) before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flarepp {

enum Dtype { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Split-N encoder partials (synthesis and encode steps).
struct EncodeParams {
  const void* q;          // qscale == 0: latent operand [.., Mpad, D] (dtype, or fp32 on
                          // the fp32 path), prescaled by scale*log2(e), padded rows zero;
                          // qscale > 0: the caller's latents [.., M, D] unscaled
  int64_t q_b_stride;     // elements between batch elements (0 = shared)
  int64_t q_h_stride;     // elements between heads
  float qscale;           // > 0: form the operand (dtype)(qscale * q) on load
  const void* k;          // [B, H, N, D]
  const void* v;          // [B, H, N, D]; may equal k
  int B, H;
  int64_t N;
  int M, Mpad;
  int64_t chunk_tokens;   // multiple of 64
  int nchunks;
  const float* gate;      // non-null: skip heads whose sigma(gate) == 0
  float* part_m;          // [B*H, nchunks, Mpad] reference (base-2 units)
  float* part_l;          // [B*H, nchunks, Mpad] sum of 2^(s - m)
  float* part_o;          // [B*H, nchunks, Mpad, D] unnormalised outputs
};

// Merge of the partials plus the gated query update, or plain operand prep.
struct CombineParams {
  int B, H, M, Mpad, D;
  int nsets;              // latent sets written: B*H (per batch) or H (shared)
  int nchunks;            // 0: no partials
  const float* part_m;
  const float* part_l;
  const float* part_o;
  int mode;               // kModeQuery or kModeValue
  // query mode: q = fixed + sigma * merged (sigma = 0 -> q = fixed, partials unread)
  const void* fixed;      // [.., H, M, D] in dtype `fixed_dtype`, or null
  int64_t fixed_b_stride; // elements between batch elements of `fixed` (0 = shared)
  int fixed_dtype;
  const float* gate;      // gate logits [H]; null with force_fixed -> sigma = 0
  int force_fixed;        // 1: ignore partials, q = fixed
  float cscale;           // operand prescale scale*log2(e)
  // value mode: z = merged, or z = z_in when nchunks == 0
  const float* z_in;      // [B*H, M, D] fp32, or null
  float* z_out;           // [B*H, M, D] fp32, or null
  // saved for the backward pass (all optional, fp32, natural [sets][M][D] or [sets][M]):
  float* q_out;           // query mode: q = fixed + sigma * merged, unscaled
  float* dyn_out;         // query mode: merged (q_dyn), 0 where sigma == 0
  float* lse_out;         // log2 of the merged row sum plus its reference (base 2)
  // operand written for the next step
  void* out;
  int out_kind;           // kOutNatural (dtype [sets][Mpad][D]), kOutNatural32 (fp32
                          // [sets][Mpad][D]); rows m >= M are written as zeros
  int out_dtype;
  int lanes_log2;         // set by launch_combine: log2 of the lanes merging one slot
};
enum { kModeQuery = 0, kModeValue = 1 };
enum { kOutNatural = 0, kOutNatural32 = 2 };

// Decoder: y = softmax over latents of (k q^T) applied to z.
struct DecodeParams {
  const void* q;          // latent operand [.., Mpad, D] (prescaled), or with qscale > 0
                          // the caller's latents [.., M, D] unscaled
  int64_t q_b_stride, q_h_stride;
  float qscale;           // > 0: form the operand (dtype)(qscale * q) on load
  const void* zt;         // value operand [B*H][Mpad][D]: dtype, or fp32 on the fp32
                          // path; rows m >= M zero
  const void* k;          // [B, H, N, D]
  void* y;                // [B, H, N, D]
  float* lse_out;         // optional [B*H, N]: per token log2(row sum) + reference
  unsigned long long* redo;  // per (workgroup, wave): tiles needing the exact path
  int B, H;
  int64_t N;
  int M, Mpad;
  int wg_per_bh;
};

hipError_t launch_encode(int dtype, int D, const EncodeParams& p, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
hipError_t launch_decode(int dtype, int D, const DecodeParams& p, hipStream_t s);

// Launch-shape helpers shared with the workspace sizing.
int encode_waves(int M);                 // waves per encoder workgroup
int encode_tile_tokens();                // tokens per encoder LDS tile
int latent_pad(int M, int dtype);        // Mpad
int decode_lds_bytes(int M, int D, int dtype);
int decode_tokens_per_tile(int D);       // tokens per decoder workgroup iteration
int decode_waves(int D);                 // waves per decoder workgroup

}  // namespace flarepp
