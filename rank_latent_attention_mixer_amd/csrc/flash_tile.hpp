// Wave-level online-softmax attention on the gfx950 matrix cores.
//
// One wave owns NC blocks of 32 query columns r (the "register side": the
// latents in the encoder, the tokens in the decoder) and consumes keys in
// groups of 32 (the "streamed side").  For every column it keeps
//   ref  - a reference m (base-2 score units), held negated and replicated
//          so that it is the C operand of the score product, which then
//          returns S' - m with no VALU subtraction;
//   lsum - this lane's share of sum_j 2^(S'_j - m);
//   o    - O^T[d][r] = sum_j 2^(S'_j - m) V[j][d]  (fp32 accumulators).
// Scores S' are already in base-2 units: the caller folds scale * log2(e)
// into the latent operand, so p = v_exp_f32(S' - m).
//
// The reference is set once, to the exact column maximum of the first key
// group, and never moves: the normalised result sum_j p_j v_j / sum_j p_j
// does not depend on m, and in floating point only overflow could go wrong
// -- a later score exceeding the reference by more than the range of the
// probability type (2^127 for bf16, 2^15 for fp16) or the fp32 sums.  Such
// inputs are detected once per column at the end (a non-finite l or O) and
// the caller recomputes that wave's columns with the exact two-pass method
// (global maximum first, then the sums).  The steady state therefore has no
// branch, no maximum and no rescale: per 32 x 32 score block it issues 16
// v_exp_f32, 8 v_cvt_pk and 8 v_dot2 next to four matrix-core ops.
//
// Sources for the operation: FLARE.py README, "FLARE++" and "FLARE"
// listings (scaled-dot-product attention); the per-chunk statistics
// (m, l, O) follow issue #2024, "Multi-GPU context parallelism" (latent-sized
// outputs plus log-sum-exp statistics per token shard).
#pragma once

#include <type_traits>

#include "flarepp_device.hpp"

namespace flarepp {

// compile-time integer argument for generic lambdas
template <int V>
using IntC = std::integral_constant<int, V>;

template <typename T, int D, int NC>
struct FlashTile {
  static constexpr int DK = D < 16 ? 16 : D;   // contraction length of the score product
  static constexpr int KD = DK / 16;           // K=16 steps of the score product
  static constexpr int DV = D < 32 ? 32 : D;   // value rows, padded to a 32-row block
  static constexpr int NDB = DV / 32;          // 32-row blocks of O^T
  typedef typename Pack8<T>::type V8;

  V8 q[NC][KD];
  f32x16 o[NDB][NC];
  f32x16 negm[NC];
  float lsum[NC];

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) negm[cb][v] = 0.f;
      lsum[cb] = 0.f;
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
      s[cb] = mfma_32x32x16(kop[0], q[cb][0], negm[cb]);
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
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      negm[cb] -= delta[cb];
      s[cb] -= delta[cb];
    }
  }

  // p = 2^s packed as the B operands of the two K=16 steps of the P.V
  // product, the rounded values summed into lsum, then O += V^T P^T.
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
        p[cb][kk] = pack8<T>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        float acc = lsum[cb];
        acc = pair_sum(__builtin_shufflevector(p[cb][kk], p[cb][kk], 0, 1), acc);
        acc = pair_sum(__builtin_shufflevector(p[cb][kk], p[cb][kk], 2, 3), acc);
        acc = pair_sum(__builtin_shufflevector(p[cb][kk], p[cb][kk], 4, 5), acc);
        acc = pair_sum(__builtin_shufflevector(p[cb][kk], p[cb][kk], 6, 7), acc);
        lsum[cb] = acc;
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        o[db][cb] = mfma_32x32x16(vop[db][0], p[cb][0], o[db][cb]);
        o[db][cb] = mfma_32x32x16(vop[db][1], p[cb][1], o[db][cb]);
      }
  }

  // First group of a sweep: scores were computed with m = 0; the reference
  // becomes the group's exact column maximum.
  template <bool MASKED>
  __device__ __forceinline__ void first(f32x16 (&s)[NC], const V8 (&vop)[NDB][2], int kvalid,
                                        int h) {
    if constexpr (MASKED) mask(s, kvalid, h);
    float mx[NC];
    colmax(s, mx);
    set_reference(s, mx);
    accumulate(s, vop);
  }

  template <bool MASKED>
  __device__ __forceinline__ void next(f32x16 (&s)[NC], const V8 (&vop)[NDB][2], int kvalid,
                                       int h) {
    if constexpr (MASKED) mask(s, kvalid, h);
    accumulate(s, vop);
  }

  // True (wave-uniform) if any column of the wave ended with a non-finite
  // sum or output, i.e. the fixed reference was exceeded beyond range.
  __device__ __forceinline__ bool overflowed() const {
    bool bad = false;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      bad = bad || !__builtin_isfinite(lsum[cb]);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) bad = bad || !__builtin_isfinite(o[db][cb][v]);
    }
    return __builtin_amdgcn_ballot_w64(bad) != 0ull;
  }

  // Full row sum of column cb (the two lanes sharing the column).
  __device__ __forceinline__ float row_sum(int cb) const {
    return lsum[cb] + __shfl_xor(lsum[cb], 32);
  }
};

}  // namespace flarepp
