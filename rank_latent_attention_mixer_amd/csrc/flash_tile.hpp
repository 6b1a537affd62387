// Wave-level softmax attention on the gfx950 matrix cores.
//
// One wave owns NC blocks of 32 query columns r (the "register side": the
// latents in the encoder, the tokens in the decoder) and consumes keys in
// groups of 32 (the "streamed side").  Per column it accumulates
//   l - sum_j 2^(S'_j - m)                    (fp32, on the matrix cores)
//   o - O^T[d][r] = sum_j 2^(S'_j - m) V[j][d]  (fp32 accumulators)
// for a reference m that never moves during a sweep.  Scores S' are already
// in base-2 units: the caller folds scale * log2(e) into the latent operand,
// so p = v_exp_f32(S' - m).
//
// The normalised result sum_j p_j v_j / sum_j p_j does not depend on m; m
// only has to keep p inside the range of the probability type.
//   * bf16 probabilities share fp32's exponent range, so m = 0 is used and
//     no maximum is ever taken (REF = false).
//   * fp16 probabilities (at most 2^15.9) take m = the exact column maximum
//     of the first key group, held negated and replicated as the C operand
//     of the score product, which then returns S' - m with no VALU work
//     (REF = true).
// A column whose sums come out non-finite, or (m = 0) so small that
// probabilities may have left the normal range, is recomputed by the caller
// with the exact two-pass method (true maximum first, then the sums).  The
// steady state therefore has no branch, no maximum and no rescale: per
// 32 x 32 score block a lane issues 16 v_exp_f32 and 4 packing ops per 8
// probabilities (v_perm_b32, see pack_probs) next to two score, two P.V and
// two row-sum matrix-core ops.
//
// Row sums: summing the packed probabilities with v_dot2 forms a serial
// chain of 8 dependent VALU ops per block.  Instead each packed operand is
// also fed to a 16x16x32 matrix-core op whose A operand is a fixed 0/1
// pattern: in that op's B layout lane l holds k-group l/16 = 2(l/32) + r/16
// of column l%16, so row 0 of the pattern (ones on k-groups 0 and 2) sums
// the 16 key slots of columns 0..15 and row 1 (k-groups 1 and 3) those of
// columns 16..31.  Result row i of column n sits in lane n, element i.
//
// Sources for the operation: FLARE.py README, "FLARE++" and "FLARE"
// listings (scaled-dot-product attention); the per-chunk statistics
// (m, l, O) follow issue #2024, "Multi-GPU context parallelism" (latent-sized
// outputs plus log-sum-exp statistics per token shard).
#pragma once

#include <type_traits>
#include <utility>

#include "flarepp_device.hpp"

namespace flarepp {

// compile-time integer argument for generic lambdas
template <int V>
using IntC = std::integral_constant<int, V>;

// f(IntC<0>{}), f(IntC<1>{}), ..., f(IntC<N-1>{})
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(IntC<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T> struct ProbTraits;
template <> struct ProbTraits<__bf16> {
  static constexpr bool kRef = false;
  static constexpr unsigned kOnePair = 0x3F803F80u;  // two bf16 1.0
};
template <> struct ProbTraits<_Float16> {
  static constexpr bool kRef = true;
  static constexpr unsigned kOnePair = 0x3C003C00u;  // two fp16 1.0
};

// Smallest row sum accepted with m = 0: below it the largest probability of
// the column may be near the bottom of the normal range.
constexpr float kMinRowSum = 0x1p-80f;

template <typename T, int D, int NC, bool REF = ProbTraits<T>::kRef>
struct FlashTile {
  static constexpr int DK = D < 16 ? 16 : D;   // contraction length of the score product
  static constexpr int KD = DK / 16;           // K=16 steps of the score product
  static constexpr int DV = D < 32 ? 32 : D;   // value rows, padded to a 32-row block
  static constexpr int NDB = DV / 32;          // 32-row blocks of O^T
  static constexpr bool kRef = REF;
  typedef typename Pack8<T>::type V8;

  V8 q[NC][KD];
  f32x16 o[NDB][NC];
  f32x16 negm[REF ? NC : 1];  // -m, replicated (REF only)
  f32x4 lacc[NC];             // row sums, see header
  V8 sum_op;                  // 0/1 pattern, A operand of the row-sum product

  __device__ __forceinline__ void reset() {
    const int lane = __lane_id();
    const bool on = lane == 0 || lane == 32 || lane == 17 || lane == 49;
    const unsigned w = on ? ProbTraits<T>::kOnePair : 0u;
    sum_op = bitcast_u4<V8>(u32x4{w, w, w, w});
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      if constexpr (REF) {
#pragma unroll
        for (int v = 0; v < 16; ++v) negm[cb][v] = 0.f;
      }
      lacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][cb][v] = 0.f;
    }
  }

  // Score product of one key group: s[cb] = K . Q[cb]^T - m[cb]
  // (kop[kd]: A operand, key lane%32, d = 16kd + 8h ..).
  __device__ __forceinline__ void scores(const V8 (&kop)[KD], f32x16 (&s)[NC]) const {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      if constexpr (REF) {
        s[cb] = mfma_32x32x16(kop[0], q[cb][0], negm[cb]);
      } else {
        s[cb] = mfma_32x32x16(kop[0], q[cb][0], f32x16{});
      }
#pragma unroll
      for (int kd = 1; kd < KD; ++kd) s[cb] = mfma_32x32x16(kop[kd], q[cb][kd], s[cb]);
    }
  }

  // Keys j >= kvalid of the group get probability 0.
  __device__ __forceinline__ static void mask(f32x16 (&s)[NC], int kvalid, int h) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = 8 * (v >> 2) + 4 * h + (v & 3);
      if (j >= kvalid) {
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) s[cb][v] = -__builtin_inff();
      }
    }
  }

  // Column maximum of a group's scores (the two lanes of a column combined).
  __device__ __forceinline__ static void colmax(const f32x16 (&s)[NC], float (&mx)[NC]) {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      float m = s[cb][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) m = fmaxf(m, s[cb][v]);
      mx[cb] = fmaxf(m, __shfl_xor(m, 32));
    }
  }

  // Moves the reference by delta (scores s computed against the old one).
  __device__ __forceinline__ void set_reference(f32x16 (&s)[NC], const float (&delta)[NC]) {
    static_assert(REF, "reference only kept with REF");
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      negm[cb] -= delta[cb];
      s[cb] -= delta[cb];
    }
  }

  // p = 2^s packed as the B operands of the two K=16 steps of the P.V
  // product; O += V^T P^T and l += 1^T P^T on the matrix cores.
  //   vop[db][kk] : A operand of the P.V product, value rows of block db,
  //                 key slots 16kk + 8h .. (see flarepp_device.hpp)
  __device__ __forceinline__ void accumulate(const f32x16 (&s)[NC], const V8 (&vop)[NDB][2]) {
    V8 p[NC][2];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = __builtin_amdgcn_exp2f(s[cb][8 * kk + t]);
        p[cb][kk] = pack_probs<T>(e);
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        o[db][cb] = mfma_32x32x16(vop[db][0], p[cb][0], o[db][cb]);
        o[db][cb] = mfma_32x32x16(vop[db][1], p[cb][1], o[db][cb]);
      }
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      lacc[cb] = mfma_16x16x32(sum_op, p[cb][0], lacc[cb]);
      lacc[cb] = mfma_16x16x32(sum_op, p[cb][1], lacc[cb]);
    }
  }

  // First group of a sweep.  REF: the scores were computed with m = 0 and
  // the reference becomes the group's exact column maximum.
  template <bool MASKED>
  __device__ __forceinline__ void first(f32x16 (&s)[NC], const V8 (&vop)[NDB][2], int kvalid,
                                        int h) {
    if constexpr (MASKED) mask(s, kvalid, h);
    if constexpr (REF) {
      float mx[NC];
      colmax(s, mx);
      set_reference(s, mx);
    }
    accumulate(s, vop);
  }

  template <bool MASKED>
  __device__ __forceinline__ void next(f32x16 (&s)[NC], const V8 (&vop)[NDB][2], int kvalid,
                                       int h) {
    if constexpr (MASKED) mask(s, kvalid, h);
    accumulate(s, vop);
  }

  // Full row sum of this lane's column r = lane % 32 of block cb.
  __device__ __forceinline__ float row_sum(int cb) const {
    const int lane = __lane_id();
    const float lo = __shfl(lacc[cb][0], lane & 15);  // columns 0..15
    const float hi = __shfl(lacc[cb][1], lane & 15);  // columns 16..31
    return (lane & 16) ? hi : lo;
  }

  // Reference m of column block cb (base-2 units).
  __device__ __forceinline__ float reference(int cb) const {
    if constexpr (REF) return -negm[cb][0];
    else return 0.f;
  }

  // True (wave-uniform) if any column of the wave needs the exact two-pass
  // recompute: a non-finite sum or output, or (m = 0) a row sum so small
  // that its probabilities may have been flushed or lost precision.
  __device__ __forceinline__ bool overflowed() const {
    bool bad = false;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const float l = row_sum(cb);
      bad = bad || !__builtin_isfinite(l);
      if constexpr (!REF) bad = bad || !(l >= kMinRowSum);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) bad = bad || !__builtin_isfinite(o[db][cb][v]);
    }
    return __builtin_amdgcn_ballot_w64(bad) != 0ull;
  }

  // The same test when every value row v is bounded, |v| <= vmax: the
  // accumulators are sums of probabilities times values, so |o| <= l vmax
  // and a row sum l with l vmax < 2^126 (and l >= kMinRowSum without a
  // reference) implies finite accumulators.  With a reference the
  // probabilities are at most 65504 (fp16) and the values fp16, so a finite
  // l already bounds |o| far below the fp32 range.  NaN in l or vmax fails
  // the comparisons and counts as overflow.
  __device__ __forceinline__ bool overflowed_bounded(float vmax) const {
    bool bad = false;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const float l = row_sum(cb);
      if constexpr (REF) bad = bad || !__builtin_isfinite(l);
      else bad = bad || !(l >= kMinRowSum) || !(l * vmax < 0x1p126f);
    }
    return __builtin_amdgcn_ballot_w64(bad) != 0ull;
  }
};

}  // namespace flarepp
