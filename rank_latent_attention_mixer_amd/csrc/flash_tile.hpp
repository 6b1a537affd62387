// Wave-level online-softmax attention step on the gfx950 matrix cores.
//
// One wave owns NC blocks of 16 query columns r (the "register side": the
// latents in the encoder, the tokens in the decoder) and consumes keys in
// groups of 32 (the "streamed side").  For every column it keeps
//   ref  - the running reference m (base-2 score units); held negated and
//          replicated four times so that it can be the C operand of the
//          score product, which then returns S' - m directly;
//   lsum - this lane's share of sum_j 2^(S'_j - m);
//   o    - O^T[d][r] = sum_j 2^(S'_j - m) V[j][d]  (fp32 accumulators).
// Scores S' are already in base-2 units: the caller folds scale * log2(e)
// into the latent operand, so p = v_exp_f32(S' - m).
//
// The reference moves lazily: a group whose per-lane probability sum stays
// below 2^8 is accepted as is (every p <= 2^8, so nothing can overflow and
// no row maximum is needed).  Otherwise, and for the very first group, the
// wave takes a slow path that finds the exact column maximum of the group,
// moves the reference up to it and rescales the accumulators.  The result
// is the same normalised softmax as with an eager running maximum; only the
// intermediate scaling differs.
//
// Sources for the operation: FLARE.py README, "FLARE++" and "FLARE"
// listings (scaled-dot-product attention); the chunked statistics
// (m, l, O) follow issue #2024, "Multi-GPU context parallelism" (latent-sized
// outputs plus log-sum-exp statistics per token shard).
#pragma once

#include "flarepp_device.hpp"

namespace flarepp {

template <typename T, int D, int NC>
struct FlashTile {
  static constexpr int KD = (D + 31) / 32;      // K=32 slices of the score product
  static constexpr int DV = D < 16 ? 16 : D;    // value rows, padded to a 16-row block
  static constexpr int NDB = DV / 16;           // 16-row blocks of O^T
  typedef typename Pack8<T>::type V8;
  typedef typename Pack8<T>::pair V2;

  V8 q[NC][KD];
  f32x4 o[NDB][NC];
  f32x4 negm[NC];
  float lsum[NC];
  bool first;

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      negm[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      lsum[cb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    first = true;
  }

  // p = 2^s for the 8 scores of a column, packed as the B operand of the
  // P.V product; ts = this lane's sum of the packed (rounded) values.
  __device__ __forceinline__ static void exp_pack(const f32x4 (&s)[2][NC], V8 (&p)[NC],
                                                  float (&ts)[NC]) {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = __builtin_amdgcn_exp2f(s[0][cb][i]);
        e[4 + i] = __builtin_amdgcn_exp2f(s[1][cb][i]);
      }
      p[cb] = pack8<T>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      float acc = 0.f;
      acc = pair_sum(__builtin_shufflevector(p[cb], p[cb], 0, 1), acc);
      acc = pair_sum(__builtin_shufflevector(p[cb], p[cb], 2, 3), acc);
      acc = pair_sum(__builtin_shufflevector(p[cb], p[cb], 4, 5), acc);
      acc = pair_sum(__builtin_shufflevector(p[cb], p[cb], 6, 7), acc);
      ts[cb] = acc;
    }
  }

  // Consume one group of 32 keys.
  //   kop[jb][kd] : A operand of the score product, keys 16*jb + (lane%16)
  //   vop[db]     : A operand of the P.V product, value rows of block db in
  //                 key-slot order (see flarepp_device.hpp)
  //   kvalid      : number of valid keys in the group (1..32); the others
  //                 get probability 0
  //   g           : lane / 16
  __device__ __forceinline__ void step(const V8 (&kop)[2][KD], const V8 (&vop)[NDB], int kvalid,
                                       int g) {
    f32x4 s[2][NC];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        s[jb][cb] = mfma_16x16x32(kop[jb][0], q[cb][0], negm[cb]);
#pragma unroll
        for (int kd = 1; kd < KD; ++kd) s[jb][cb] = mfma_16x16x32(kop[jb][kd], q[cb][kd], s[jb][cb]);
      }
    }
    if (kvalid < 32) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * jb + 4 * g + i;
          if (j >= kvalid) {
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) s[jb][cb][i] = -__builtin_inff();
          }
        }
    }
    V8 p[NC];
    float ts[NC];
    exp_pack(s, p, ts);
    bool need = first;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) need = need || (ts[cb] > kTauSum);
    if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
      // slow path: move each column's reference to the group's maximum
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        float mx = s[0][cb][0];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[jb][cb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float delta = first ? mx : fmaxf(mx, 0.f);
        if (!first) {
          const float sc = __builtin_amdgcn_exp2f(-delta);
          lsum[cb] *= sc;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db][cb] *= sc;
        }
        negm[cb] -= delta;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) s[jb][cb] -= delta;
      }
      exp_pack(s, p, ts);
      first = false;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) o[db][cb] = mfma_16x16x32(vop[db], p[cb], o[db][cb]);
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) lsum[cb] += ts[cb];
  }

  // Full row sum of column cb (the four lanes sharing the column).
  __device__ __forceinline__ float row_sum(int cb) const {
    float t = lsum[cb];
    t += __shfl_xor(t, 16);
    t += __shfl_xor(t, 32);
    return t;
  }
};

}  // namespace flarepp
