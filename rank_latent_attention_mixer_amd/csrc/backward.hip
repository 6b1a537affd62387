// Backward pass of the FLARE++ and FLARE mixers on the gfx950 matrix cores.
//
// The pages define the forward pass (FLARE.py README, "FLARE++" and "FLARE"
// listings) and say the token-sharded encoder has a custom backward (issue
// #2024, "Multi-GPU context parallelism"); the gradients here follow from
// the forward by the chain rule.  For one attention O = A V with
// A = softmax_rows(s Q K^T): dV = A^T dO, dS = A * (dO V^T - rowsum(dO*O)),
// dQ = s dS K, dK = s dS^T Q.
//
// Both attentions of the encode-decode pair share one score matrix: with
// c = s log2(e) and S'[n][m] = c k_n . q_m, the decoder's weights are
// A2 = 2^(S' - lse2_n) (normalised over the latents of token n) and the
// encoder's A1 = 2^(S' - lse1_m) (over the tokens of latent m), lse being the
// base-2 log-sum-exp rows the training forward saved.  Every pass recomputes
// S' on the matrix cores with minus the lse in the product's accumulator
// input (a per-lane splat when the softmax row runs along the lane's own
// column, a per-element vector read from LDS when it runs along the rows),
// so P = 2^(S) is the normalised weight without extra VALU work.  The
// softmax-Jacobian term enters the same way: G = a . b - Delta is formed in
// fp32 inside the second product before it is rounded to an operand, so
// dS = P G never cancels in low precision.  Weights normalised over the N
// tokens (A1 and the synthesis A0) carry a factor 2^shift, undone in fp32,
// and the latent-side gradient operands are divided by a power of two per
// (b, h) that brings their largest element near 1, so fp16 operands stay
// normal numbers; the factors are undone in fp32.
//
// Two kernels, each used for several passes:
//  * bwd_lat_kernel -- latents in registers (32 per wave), tokens streamed
//    through LDS: sums over tokens (dz, dq, dq0), as split-N partials;
//  * bwd_tok_kernel -- tokens in registers, all latents resident in LDS:
//    per-token results (dk, dv, dk0).
// Per 32 x 32 block: a score product, a second product G, P = 2^S,
// T = P * G (= dS), and P.V-style products accumulating over the block's
// keys with P or T as the B operand.
#include <cmath>
#include <type_traits>

#include "backward.hpp"
#include "flash_tile.hpp"

#ifndef FLAREPP_BWD_TOK_DEFER
#define FLAREPP_BWD_TOK_DEFER 1
#endif

namespace flarepp {

namespace {

// Row-major [row][d] tensor in LDS: rows of 2*D bytes, the 16-byte chunks of
// row `row` XOR-permuted by swz(row) (row reads of 16 rows x 16 bytes and the
// transposing reads both hit distinct banks).  For D >= 16 the swizzle of row
// 32*g + r equals that of r, so a 32-row group is an immediate offset.
template <int D>
struct RowLayout {
  static constexpr int ROWB = 2 * D;
  static constexpr int CPR = D / 8;
  static constexpr int RPB = 256 / ROWB;
  __device__ __forceinline__ static int swz(int row) { return (row / RPB) % CPR; }
  __device__ __forceinline__ static int offset(int row, int byte) {
    return row * ROWB + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
  }
};

// Lane addresses of the two operand reads of a row-major LDS tensor.
template <typename T, int D>
struct LdsOps {
  using L = RowLayout<D>;
  typedef typename Pack8<T>::type V8;
  static constexpr int KD = D / 16;
  static constexpr int DV = D < 32 ? 32 : D;
  static constexpr int NDB = DV / 32;
  int kaddr[KD];
  int vaddr[NDB][2];

  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, r = lane & 31;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) kaddr[kd] = L::offset(r, 2 * (16 * kd + 8 * h));
    // transposing read: in each 16-lane group, source lane 4k+q addresses
    // row k, columns d0+4q..+3; lane j receives column d0+j of rows 0..3
    const int tr_k = (lane & 15) >> 2, tr_q = lane & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * tr_q;
      if (d >= D) d = 0;  // feeds only padded output rows
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) vaddr[db][aa] = L::offset(8 * aa + 4 * h + tr_k, 2 * d);
    }
  }
  // A operand of a product contracting over d: rows 32*grp + lane%32.
  __device__ __forceinline__ void rows(const unsigned char* base, int grp, V8 (&op)[KD]) const {
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      op[kd] = *reinterpret_cast<const V8*>(base + kaddr[kd] + grp * 32 * L::ROWB);
  }
  // A operand of a product contracting over the rows of group grp (in the
  // key-slot order of the score layout): value rows d, two K=16 steps.
  __device__ __forceinline__ void cols(const unsigned char* base, int grp,
                                       V8 (&op)[NDB][2]) const {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        short4v part[2];
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
          part[aa] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4v*)(base + vaddr[db][aa] +
                                                           (32 * grp + 16 * kk) * L::ROWB));
        op[db][kk] = __builtin_bit_cast(V8, short8v{part[0][0], part[0][1], part[0][2], part[0][3],
                                                    part[1][0], part[1][1], part[1][2], part[1][3]});
      }
  }
};

template <typename V8, int KD>
__device__ __forceinline__ void load_row_op(const void* base, int64_t row, int D, int h,
                                            V8 (&op)[KD]) {
  const unsigned char* p = reinterpret_cast<const unsigned char*>(base);
#pragma unroll
  for (int kd = 0; kd < KD; ++kd)
    op[kd] = bitcast_u4<V8>(ldg16(p + (row * D + 16 * kd + 8 * h) * 2));
}

template <typename V8, int KD>
__device__ __forceinline__ f32x16 product(const V8 (&a)[KD], const V8 (&b)[KD], f32x16 c) {
#pragma unroll
  for (int kd = 0; kd < KD; ++kd) c = mfma_32x32x16(a[kd], b[kd], c);
  return c;
}

__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 v;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = x;
  return v;
}

// Slots j >= kvalid of a 32-key group get probability 0.
__device__ __forceinline__ void mask_slots(f32x16& s, int kvalid, int h) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int j = 8 * (v >> 2) + 4 * h + (v & 3);
    if (j >= kvalid) s[v] = -__builtin_inff();
  }
}

// Per-element C operand from a float vector in LDS: element v of the lane
// belongs to row 32 grp + 8 (v / 4) + 4 h + v % 4 of the score layout.
__device__ __forceinline__ f32x16 lds_rowvec(const float* vec, int grp, int h) {
  f32x16 c;
#pragma unroll
  for (int aa = 0; aa < 4; ++aa) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(vec + 32 * grp + 8 * aa + 4 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) c[4 * aa + i] = x[i];
  }
  return c;
}

// Pack 16 accumulator values as the two K=16 B operands of a product over
// the group's rows (round to nearest even).
template <typename T>
__device__ __forceinline__ void pack16(const float (&v)[16], typename Pack8<T>::type (&op)[2]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    op[kk] = pack8<T>(v[8 * kk], v[8 * kk + 1], v[8 * kk + 2], v[8 * kk + 3], v[8 * kk + 4],
                      v[8 * kk + 5], v[8 * kk + 6], v[8 * kk + 7]);
}

template <typename V8, int NDB>
__device__ __forceinline__ void accumulate(f32x16 (&acc)[NDB], const V8 (&a)[NDB][2],
                                           const V8 (&p)[2]) {
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    acc[db] = mfma_32x32x16(a[db][0], p[0], acc[db]);
    acc[db] = mfma_32x32x16(a[db][1], p[1], acc[db]);
  }
}

// Accumulator rows d = 32db + 8a + 4h + i of column lane%32, as float4 runs;
// with add set, added to what dst holds.
template <int D, int NDB>
__device__ __forceinline__ void store_acc_row(float* dst, const f32x16 (&acc)[NDB], int h,
                                              float scale, int add = 0) {
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const int d0 = 32 * db + 8 * aa + 4 * h;
      if (d0 < D) {
        f32x4 v = f32x4{acc[db][4 * aa] * scale, acc[db][4 * aa + 1] * scale,
                        acc[db][4 * aa + 2] * scale, acc[db][4 * aa + 3] * scale};
        if (add) v += *reinterpret_cast<const f32x4*>(dst + d0);
        *reinterpret_cast<f32x4*>(dst + d0) = v;
      }
    }
}

// Dot product of two 16-byte chunks of 8 operand values: four two-term dot
// instructions, fp32 accumulation (each product of two 16-bit values is
// exact in fp32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, int dtype) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // elements copied out first: a bit cast of a vector element expression
    // itself reads the vector's first element whatever the index
    const unsigned x = a[j], y = b[j];
    acc = dtype == kBF16
              ? __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                                __builtin_bit_cast(bf16x2_t, y), acc, false)
              : __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x),
                                       __builtin_bit_cast(f16x2_t, y), acc, false);
  }
  return acc;
}

// v plus the value of lane ^ 1 (and, with x2, of lane ^ 2) within each quad.
__device__ __forceinline__ float quad_xor_add(float v, bool x2) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
  if (x2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));
  return v;
}

// ---------------------------------------------------------------------------
// Latents in registers, tokens streamed through LDS.
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 8;
constexpr int kBwdTile = 128;  // tokens per LDS tile

// Waves (32 latents each) per latent-pass workgroup: 16 where the kernel
// fits 128 VGPRs (four waves per SIMD, each token tile shared by twice the
// latents), 8 at D = 64.
template <int D>
constexpr int lat_waves() { return D <= 32 ? 16 : 8; }

// Whether the decoder's latent pass forms -Delta2 itself: its tile staging
// (one 16-byte chunk per thread) leaves at least as many threads idle as
// it uses.
template <int D>
constexpr bool lat_forms_delta2() { return 2 * kBwdTile * RowLayout<D>::CPR <= 64 * lat_waves<D>(); }

template <typename T, int D, int MODE>
__global__ __launch_bounds__(64 * lat_waves<D>()) void bwd_lat_kernel(BwdLatParams a) {
  constexpr int NWV = lat_waves<D>();
  using O = LdsOps<T, D>;
  using V8 = typename O::V8;
  using L = RowLayout<D>;
  constexpr int KD = O::KD, NDB = O::NDB;
  constexpr bool DEC = MODE == kBwdLatDec;
  constexpr int NT = MODE == kBwdLatSyn ? 1 : 2;
  constexpr int GI = NT - 1;                 // token tensor of the G product
  constexpr int TB = kBwdTile * L::ROWB;     // bytes per tile per tensor
  constexpr int NV = DEC ? kBwdTile : 4;     // per-token C values per tile
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][NT * TB];
  __shared__ __attribute__((aligned(16))) float tvec[2][2][NV];  // -lse2, -Delta2

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int set = blockIdx.x / a.nchunks;
  const int chunk = blockIdx.x - set * a.nchunks;
  const int b = set / a.H, hd = set - b * a.H;
  // closed gate (synthesis pass): the partials of this head are zero
  const bool closed = a.gate != nullptr && gate_sigma(a.gate[hd]) == 0.f;
  const int col = blockIdx.y * 32 * NWV + wave * 32 + r;            // latent of this lane
  const int colc = min(col, a.M - 1);

  V8 qop[KD], gop[KD];
  load_row_op<V8, KD>(reinterpret_cast<const unsigned char*>(a.qop) +
                          2 * (b * a.q_b_stride + hd * a.q_h_stride),
                      colc, D, h, qop);
  load_row_op<V8, KD>(reinterpret_cast<const unsigned char*>(a.gop) +
                          2 * ((int64_t)set * a.Mpad * D),
                      colc, D, h, gop);
  f32x16 cs = splat16(0.f), cg = splat16(0.f);
  if constexpr (!DEC) {
    cs = splat16(a.shift - a.lse[(int64_t)set * a.M + colc]);
    cg = splat16(a.negg[(int64_t)set * a.M + colc]);
  }

  O ops;
  ops.init(lane);
  f32x16 y[NDB], x[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    y[db] = splat16(0.f);
    x[db] = splat16(0.f);
  }

  const int64_t n0 = (int64_t)chunk * a.chunk_tokens;
  const int ntok = (int)(min(a.N, n0 + a.chunk_tokens) - n0);
  const int ntiles = closed ? 0 : (ntok + kBwdTile - 1) / kBwdTile;
  const unsigned char* tbase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    tbase[t] = reinterpret_cast<const unsigned char*>(a.t[t]) + ((int64_t)set * a.N + n0) * D * 2;

  // tile staging through registers: 16-byte chunks, thread-strided; the
  // rows past the chunk's end repeat its last token (their weights are 0)
  constexpr int CH = kBwdTile * L::CPR;                      // chunks per tensor per tile
  constexpr int PER = (CH + 64 * NWV - 1) / (64 * NWV);
  // Decoder: where the tile's chunks leave whole waves idle (threads CH to
  // 2 CH - 1), those waves stage the tile's dy chunks a second time with the
  // matching y chunks and form -Delta2 = -(dy . y) per token, for this
  // pass's G product and, stored, for the token pass.
  constexpr bool kDelta = lat_forms_delta2<D>() && DEC;
  constexpr int kDt = std::is_same<T, __bf16>::value ? kBF16 : kF16;
  const int e2 = tid - CH;
  const bool delta_lane = kDelta && e2 >= 0 && e2 < CH;     // wave-uniform
  const unsigned char* ybase =
      kDelta ? reinterpret_cast<const unsigned char*>(a.y_tok) + ((int64_t)set * a.N + n0) * D * 2
             : nullptr;
  u32x4 stage[NT][PER];
  float sv0 = 0.f, sv1 = 0.f;
  float lmin = __builtin_inff();  // decoder: minimum lse2 over the chunk's tokens
  auto fetch = [&](int tile) {
    const int lim = ntok - 1 - tile * kBwdTile;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = tid + i * 64 * NWV;
        if (e < CH) {
          const int row = e / L::CPR, c = e - row * L::CPR;
          stage[t][i] = ldg16(tbase[t] + ((int64_t)(tile * kBwdTile + min(row, lim)) * D + 8 * c) * 2);
        }
      }
    if (DEC && tid < kBwdTile) {
      const int64_t n = (int64_t)set * a.N + n0 + tile * kBwdTile + min(tid, lim);
      sv0 = a.tok_lse[n];
      lmin = fminf(lmin, sv0);
      if constexpr (!kDelta) sv1 = a.tok_negd[n];
    }
    if constexpr (kDelta) {
      if (delta_lane) {
        const int row = e2 / L::CPR, c = e2 - row * L::CPR;
        const int64_t off = ((int64_t)(tile * kBwdTile + min(row, lim)) * D + 8 * c) * 2;
        stage[0][0] = ldg16(tbase[1] + off);  // dy
        stage[1][0] = ldg16(ybase + off);     // y
      }
    }
  };
  auto store = [&](int buf, int tile) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = tid + i * 64 * NWV;
        if (e < CH) {
          const int row = e / L::CPR, c = e - row * L::CPR;
          *reinterpret_cast<u32x4*>(&lds[buf][t * TB + L::offset(row, 16 * c)]) = stage[t][i];
        }
      }
    if constexpr (kDelta) {
      if (delta_lane) {
        // the same chunk products and lane butterfly as the separate
        // per-token pass, so -Delta2 comes out bit for bit the same
        static_assert(L::CPR == 2 || L::CPR == 4, "one row per lane quad");
        const float v = quad_xor_add(dot8(stage[0][0], stage[1][0], kDt), L::CPR == 4);
        const int row = e2 / L::CPR;
        if (e2 - row * L::CPR == 0) {
          tvec[buf][1][row] = -v;
          if (blockIdx.y == 0 && tile * kBwdTile + row < ntok)
            a.negd_out[(int64_t)set * a.N + n0 + tile * kBwdTile + row] = -v;
        }
      }
    }
    if (DEC && tid < kBwdTile) {
      tvec[buf][0][tid] = -sv0;
      if constexpr (!kDelta) tvec[buf][1][tid] = sv1;
    }
  };

  if (ntiles > 0) {
    fetch(0);
    store(0, 0);
  }
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int cur = tile & 1;
    if (tile + 1 < ntiles) fetch(tile + 1);
    const int rem = ntok - tile * kBwdTile;
    for (int g = 0; g < kBwdTile / 32; ++g) {
      const int kvalid = min(32, rem - 32 * g);
      if (kvalid <= 0) break;  // block-uniform
      const unsigned char* base = lds[cur];
      V8 kop[KD];
      ops.rows(base, g, kop);
      f32x16 s = product<V8, KD>(kop, qop, DEC ? lds_rowvec(tvec[cur][0], g, h) : cs);
      f32x16 gg;
      if constexpr (GI == 0) {  // synthesis: the G product's token rows are the score rows
        gg = product<V8, KD>(kop, gop, cg);
      } else {
        V8 gk[KD];
        ops.rows(base + GI * TB, g, gk);
        gg = product<V8, KD>(gk, gop, DEC ? lds_rowvec(tvec[cur][1], g, h) : cg);
      }
      if (kvalid < 32) mask_slots(s, kvalid, h);
      float p[16], t[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[v] = __builtin_amdgcn_exp2f(s[v]);
        t[v] = p[v] * gg[v];
      }
      V8 Tm[2];
      pack16<T>(t, Tm);
      V8 va[NDB][2];
      ops.cols(base, g, va);
      accumulate<V8, NDB>(y, va, Tm);
      if constexpr (DEC) {
        V8 P[2];
        pack16<T>(p, P);
        ops.cols(base + TB, g, va);
        accumulate<V8, NDB>(x, va, P);
      }
    }
    if (tile + 1 < ntiles) store(cur ^ 1, tile + 1);
    __syncthreads();
  }

  if constexpr (DEC) {
    // two partial minima per chunk (the two waves that read lse2), for the
    // token pass's choice of its one-exponential form
    if (a.lse_min_out != nullptr && blockIdx.y == 0 && wave < kBwdTile / 64) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) lmin = fminf(lmin, __shfl_xor(lmin, o));
      if (lane == 0) a.lse_min_out[((int64_t)set * a.nchunks + chunk) * 2 + wave] = lmin;
    }
  }
  if (col >= a.M) return;
  const int64_t prow = ((int64_t)set * a.nchunks + chunk) * a.Mpad + col;
  store_acc_row<D, NDB>(a.part[0] + prow * D, y, h, 1.f);
  if constexpr (DEC) store_acc_row<D, NDB>(a.part[1] + prow * D, x, h, 1.f);
}

// ---------------------------------------------------------------------------
// Tokens in registers, all latents resident in LDS.
// ---------------------------------------------------------------------------
// Waves per token-pass workgroup: the workgroup holds every latent of its
// head in LDS, so it is the only one on its CU; the synthesis pass is small
// enough in registers (<= 128 VGPRs) to run four waves per SIMD.
template <int MODE, int D>
constexpr int tok_waves() { return (MODE == kBwdTokSyn && D <= 32) ? 16 : 8; }

template <typename T, int D, int MODE>
__global__ __launch_bounds__((64 * tok_waves<MODE, D>())) void bwd_tok_kernel(BwdTokParams a) {
  constexpr int NWV = tok_waves<MODE, D>();
  using O = LdsOps<T, D>;
  using V8 = typename O::V8;
  using L = RowLayout<D>;
  constexpr int KD = O::KD, NDB = O::NDB;
  constexpr bool DEC = MODE == kBwdTokFlare;  // decoder terms (P2, G1)
  // LDS, one block per group of 32 latents: the group's rows of latent
  // tensors 0 (score rows, Y columns), 1 (G1 rows) and 2 (G2 rows, X
  // columns), then its 32 entries of the per-latent vectors (C of P1, C of
  // G2, the fast form's U).  Every read of a group is one lane address plus
  // a compile-time offset from the group's base.
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  constexpr int kTen = 32 * L::ROWB;        // one tensor's rows of a group
  constexpr int kVec = 3 * kTen;            // the group's vectors, 3 x 32 floats
  constexpr int kGrp = kVec + 3 * 32 * 4;   // bytes per group

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int set = blockIdx.x / a.wg_per_bh;
  const int part = blockIdx.x - set * a.wg_per_bh;
  const int b = set / a.H, hd = set - b * a.H;
  constexpr int kTok = 32 * NWV;
  const int64_t ntiles = (a.N + kTok - 1) / kTok;
  const bool closed = a.gate != nullptr && gate_sigma(a.gate[hd]) == 0.f;

  const int Mk = (a.M + 31) & ~31;
  // per-latent vector j, entry m
  auto vec_at = [&](int j, int m) -> float& {
    return *reinterpret_cast<float*>(lds_raw + (m >> 5) * kGrp + kVec + 128 * j + 4 * (m & 31));
  };
  // FLARE part, fast form: P2 = P1 U[m] W[n] with U = 2^(lse1 - shift - Ls)
  // and W = 2^(Ls - lse2 - e) (the two weights share their score; Ls, the
  // largest lse1 - shift of the range, keeps U <= 1), one exponential per
  // pair instead of two.  Taken when W stays far inside fp32 for every token
  // of the set (else the two-exponential form).
  constexpr bool kFastForm = DEC && D <= 32;
  __shared__ float red[2][16];
  bool fast = false;
  float Ls = 0.f;
  if (!closed) {
    // resident latents: rows [0, Mk) of each tensor, rows >= M zero
    const int CH = Mk * L::CPR;
    for (int t = 0; t < 3; ++t) {
      if (a.lat[t] == nullptr) continue;
      const unsigned char* src = reinterpret_cast<const unsigned char*>(a.lat[t]) +
                                 2 * (b * a.lat_b_stride[t] + hd * a.lat_h_stride[t]);
      for (int e = tid; e < CH; e += 64 * NWV) {
        const int row = e / L::CPR, c = e - row * L::CPR;
        const u32x4 v = row < a.M ? ldg16(src + ((int64_t)row * D + 8 * c) * 2)
                                  : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&lds_raw[(row >> 5) * kGrp + t * kTen +
                                           L::offset(row & 31, 16 * c)]) = v;
      }
    }
    float lmax = -__builtin_inff(), tmin = __builtin_inff();
    for (int m = tid; m < Mk; m += 64 * NWV) {
      const bool in = m < a.M;
      const int64_t i = (int64_t)set * (a.lat_stat_stride ? a.lat_stat_stride : a.M) + m;
      vec_at(0, m) = in ? a.shift - a.lat_lse[i] : 0.f;
      vec_at(1, m) = in ? a.lat_negd[i] : 0.f;
      if (in) lmax = fmaxf(lmax, a.lat_lse[i]);
    }
    if constexpr (kFastForm) {
      for (int p = tid; p < a.lse_min_parts; p += 64 * NWV)
        tmin = fminf(tmin, a.tok_lse_min[(int64_t)set * a.lse_min_parts + p]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        lmax = fmaxf(lmax, __shfl_xor(lmax, o));
        tmin = fminf(tmin, __shfl_xor(tmin, o));
      }
      if (lane == 0) {
        red[0][wave] = lmax;
        red[1][wave] = tmin;
      }
      __syncthreads();
      lmax = red[0][0];
      tmin = red[1][0];
      for (int w = 1; w < NWV; ++w) {
        lmax = fmaxf(lmax, red[0][w]);
        tmin = fminf(tmin, red[1][w]);
      }
      Ls = lmax - a.shift;
      // log2 of the largest W; the smallest is >= -17 - e (lse2 <= log2 M +
      // the largest lse1), so bounding e bounds it too
      const float e = a.set_e[set];
      const float wmax = Ls - tmin - e;
      fast = a.tok_lse_min != nullptr && fabsf(wmax) <= 100.f && fabsf(e) <= 100.f &&
             fabsf(Ls) <= 1e30f;
      if (fast)
        for (int m = tid; m < Mk; m += 64 * NWV)
          vec_at(2, m) = m < a.M ? __builtin_amdgcn_exp2f(-vec_at(0, m) - Ls) : 0.f;
    }
  }
  __syncthreads();
  const int nfull = a.M / 32, mtail = a.M - 32 * nfull;

  O ops;
  ops.init(lane);
  const int64_t toff = (int64_t)set * a.N * D * 2;
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(a.kt) + toff;
  const unsigned char* g1g = DEC ? reinterpret_cast<const unsigned char*>(a.g1t) + toff : nullptr;
  const unsigned char* g2g = reinterpret_cast<const unsigned char*>(a.g2t) + toff;

  for (int64_t tile = part; tile < ntiles; tile += a.wg_per_bh) {
    const int64_t n = tile * kTok + wave * 32 + r;
    const int64_t nc = min(n, a.N - 1);
    float* out0 = a.out0 + ((int64_t)set * a.N + n) * D;
    float* out1 = a.out1 ? a.out1 + ((int64_t)set * a.N + n) * D : nullptr;
    if (closed) {  // the synthesis does not reach the output: zero gradient
      if (n < a.N && h == 0 && !a.accumulate)
        for (int d = 0; d < D; d += 4) {
          *reinterpret_cast<f32x4*>(out0 + d) = f32x4{0.f, 0.f, 0.f, 0.f};
          if (out1) *reinterpret_cast<f32x4*>(out1 + d) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      continue;
    }
    V8 kop[KD], b1[KD], b2[KD];
    load_row_op<V8, KD>(kg, nc, D, h, kop);
    load_row_op<V8, KD>(g2g, nc, D, h, b2);
    f32x16 cs2 = splat16(0.f), cg1 = splat16(0.f);
    float wn = 0.f;
    if constexpr (DEC) {
      load_row_op<V8, KD>(g1g, nc, D, h, b1);
      const float c2 = -a.tok_lse[(int64_t)set * a.N + nc] - a.set_e[set];
      cs2 = splat16(c2);
      wn = __builtin_amdgcn_exp2f(c2 + Ls);
      cg1 = splat16(a.tok_negd[(int64_t)set * a.N + nc]);
    }
    f32x16 y[NDB], x[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      y[db] = splat16(0.f);
      x[db] = splat16(0.f);
    }
    // Packed operands of a group whose P.V-style products are still to be
    // issued: at D <= 32 a group's accumulating products are deferred until
    // the next group's score and G products are in flight, so that the
    // matrix cores work through them while the VALU forms the next group's
    // T (same products, same order of accumulation).  Only the FLARE pass
    // at D <= 32 defers: at D = 64, and in the 16-wave synthesis pass held
    // to 128 VGPRs, the held operands would not fit the registers.
    constexpr bool kDefer = FLAREPP_BWD_TOK_DEFER && DEC && D != 64;
    V8 pend_t[2], pend_p[2];
    const unsigned char* pend_gb = lds_raw;
    auto flush = [&]() {
      V8 va[NDB][2];
      ops.cols(pend_gb, 0, va);
      accumulate<V8, NDB>(y, va, pend_t);
      ops.cols(pend_gb + 2 * kTen, 0, va);
      accumulate<V8, NDB>(x, va, pend_p);
    };
    // one group of 32 latents; the masking of a partial last group is a
    // compile-time variant, so full groups carry no selects.  FIRST: no
    // earlier group is pending.
    auto group = [&](int G, int kvalid, auto tail, auto fast_form, auto first) {
      constexpr bool FAST = decltype(fast_form)::value;
      const unsigned char* gb = lds_raw + G * kGrp;
      const float* gv = reinterpret_cast<const float*>(gb + kVec);
      V8 lop[KD];
      ops.rows(gb, 0, lop);
      f32x16 s1 = product<V8, KD>(lop, kop, lds_rowvec(gv, 0, h));
      f32x16 s2 = splat16(0.f);
      if constexpr (DEC && !FAST) s2 = product<V8, KD>(lop, kop, cs2);
      ops.rows(gb + 2 * kTen, 0, lop);
      const f32x16 g2 = product<V8, KD>(lop, b2, lds_rowvec(gv + 32, 0, h));
      f32x16 g1 = splat16(0.f);
      if constexpr (DEC) {
        ops.rows(gb + kTen, 0, lop);
        g1 = product<V8, KD>(lop, b1, cg1);
      }
      if constexpr (kDefer && !decltype(first)::value) flush();
      if constexpr (decltype(tail)::value) {
        mask_slots(s1, kvalid, h);
        if constexpr (DEC && !FAST) mask_slots(s2, kvalid, h);
      }
      float p[16], t[16];
      if constexpr (FAST) {
        // T = P1 (G2 + U W G1)
        const f32x16 u = lds_rowvec(gv + 64, 0, h);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          p[v] = __builtin_amdgcn_exp2f(s1[v]);
          t[v] = p[v] * fmaf(u[v], wn * g1[v], g2[v]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          p[v] = __builtin_amdgcn_exp2f(s1[v]);
          t[v] = p[v] * g2[v];
          if constexpr (DEC) t[v] = fmaf(__builtin_amdgcn_exp2f(s2[v]), g1[v], t[v]);
        }
      }
      if constexpr (kDefer) {
        pack16<T>(t, pend_t);
        pack16<T>(p, pend_p);
        pend_gb = gb;
      } else {
        V8 Tm[2], P[2];
        pack16<T>(t, Tm);
        pack16<T>(p, P);
        V8 va[NDB][2];
        ops.cols(gb, 0, va);
        accumulate<V8, NDB>(y, va, Tm);
        ops.cols(gb + 2 * kTen, 0, va);
        accumulate<V8, NDB>(x, va, P);
      }
    };
    if constexpr (D == 64) {  // one code path (a second one spills at this width)
      for (int G = 0; G * 32 < a.M; ++G)
        group(G, G < nfull ? 32 : mtail, std::true_type{}, std::false_type{}, std::true_type{});
    } else {
      auto groups = [&](auto fast_form) {
        if constexpr (kDefer) {
          if (nfull > 0) {
            group(0, 32, std::false_type{}, fast_form, std::true_type{});
#pragma unroll 1
            for (int G = 1; G < nfull; ++G)
              group(G, 32, std::false_type{}, fast_form, std::false_type{});
            if (mtail > 0) group(nfull, mtail, std::true_type{}, fast_form, std::false_type{});
          } else {  // M < 32: the masked group alone
            group(0, mtail, std::true_type{}, fast_form, std::true_type{});
          }
          flush();
        } else {
#pragma unroll 1
          for (int G = 0; G < nfull; ++G) group(G, 32, std::false_type{}, fast_form, std::true_type{});
          if (mtail > 0) group(nfull, mtail, std::true_type{}, fast_form, std::true_type{});
        }
      };
      if constexpr (kFastForm) {
        if (fast) groups(std::true_type{});  // block-uniform
        else groups(std::false_type{});
      } else {
        groups(std::false_type{});
      }
    }
    if (n >= a.N) continue;
    const float up = exp2f(a.set_e[set]);
    if (out1) {
      store_acc_row<D, NDB>(out0, y, h, up * a.s_over_c, a.accumulate);
      store_acc_row<D, NDB>(out1, x, h, up, a.accumulate);
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) y[db][v] = fmaf(a.s_over_c, y[db][v], x[db][v]);
      store_acc_row<D, NDB>(out0, y, h, up, a.accumulate);
    }
  }
}

// ---------------------------------------------------------------------------
// Small steps between the passes (fp32 bookkeeping; one lane per element,
// a wave per latent or token row where a dot product over d is needed).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float ld_any(const void* p, int64_t i, int dtype) {
  if (dtype == kBF16) return (float)reinterpret_cast<const __bf16*>(p)[i];
  if (dtype == kF16) return (float)reinterpret_cast<const _Float16*>(p)[i];
  return reinterpret_cast<const float*>(p)[i];
}
__device__ __forceinline__ void st_op(void* p, int64_t i, int dtype, float x) {
  if (dtype == kBF16) reinterpret_cast<__bf16*>(p)[i] = (__bf16)x;
  else reinterpret_cast<_Float16*>(p)[i] = (_Float16)x;
}

// Sum over the 64-lane wave of a value held by lanes [0, width).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// -Delta2 = -(dy . y) per token row: D/8 lanes per row, one 16-byte chunk
// each, reduced over the row's lanes.
__global__ __launch_bounds__(256) void bwd_tok_prep_kernel(BwdPrepParams a) {
  const int cpr = a.D / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = t / cpr;
  const int c = (int)(t - row * cpr);
  const bool live = row < a.rows;
  float v = 0.f;
  if (live) {
    const int64_t off = (row * a.D + 8 * c) * 2;
    v = dot8(ldg16(reinterpret_cast<const unsigned char*>(a.dy) + off),
             ldg16(reinterpret_cast<const unsigned char*>(a.y) + off), a.dtype);
  }
  for (int o = 1; o < cpr; o <<= 1) v += __shfl_xor(v, o);
  if (live && c == 0) a.negd[row] = -v;
}

// Latent rows: convert fp32 [sets][M][D] to operand rows [sets][Mpad][D]
// scaled by `scale`, rows >= M zero.
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdRowsParams a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.sets * a.Mpad * a.D;
  if (i >= total) return;
  const int64_t set = i / ((int64_t)a.Mpad * a.D);
  const int64_t rem = i - set * a.Mpad * a.D;
  const int m = (int)(rem / a.D), d = (int)(rem - (int64_t)m * a.D);
  float v = 0.f;
  if (m < a.M) v = a.scale * ld_any(a.in, (set % a.in_sets) * a.in_set_stride + (int64_t)m * a.D + d, a.in_dtype);
  st_op(a.out, i, a.dtype, v);
}

// Four lanes per output: lane q of a slot sums the chunks c = q mod 4, then
// the four combine in a fixed butterfly (every lane stays for the shuffles).
__device__ __forceinline__ float chunk_sum4(const float* part, int64_t stride, int nchunks, int q) {
  float acc = 0.f;
#pragma unroll 4
  for (int c = q; c < nchunks; c += 4) acc += part[(int64_t)c * stride];
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  return acc;
}

// After the decoder's latent pass: dq = s Y, dz = X, summed over chunks.
__global__ __launch_bounds__(256) void bwd_dec_sums_kernel(BwdSumsParams a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int q = (int)(t & 3);
  const int64_t total = (int64_t)a.sets * a.M * a.D;
  const int64_t i = min(t >> 2, total - 1);
  const int64_t set = i / ((int64_t)a.M * a.D);
  const int64_t md = i - set * a.M * a.D;
  const int m = (int)(md / a.D), d = (int)(md - (int64_t)m * a.D);
  const int64_t p = (((int64_t)set * a.nchunks) * a.Mpad + m) * a.D + d;
  const int64_t stride = (int64_t)a.Mpad * a.D;
  const float Y = chunk_sum4(a.part[0] + p, stride, a.nchunks, q);
  const float X = chunk_sum4(a.part[1] + p, stride, a.nchunks, q);
  if (q == 0 && (t >> 2) < total) {
    a.dq[i] = a.s * Y;
    a.dz[i] = X;
  }
}

// dst (+)= s 2^e * (sum over chunks of a latent pass's Y), per (set, m, d).
__global__ __launch_bounds__(256) void bwd_add_sums_kernel(BwdAddParams a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int q = (int)(t & 3);
  const int64_t total = (int64_t)a.sets * a.M * a.D;
  const int64_t i = min(t >> 2, total - 1);
  const int64_t set = i / ((int64_t)a.M * a.D);
  const int64_t md = i - set * a.M * a.D;
  const int m = (int)(md / a.D), d = (int)(md - (int64_t)m * a.D);
  const float acc = chunk_sum4(a.part + (((int64_t)set * a.nchunks) * a.Mpad + m) * a.D + d,
                               (int64_t)a.Mpad * a.D, a.nchunks, q);
  if (q == 0 && (t >> 2) < total) {
    const float f = a.s * (a.set_e ? exp2f(a.set_e[set]) : 1.f);
    a.dst[i] = a.accumulate ? a.dst[i] + f * acc : f * acc;
  }
}

// Per head: latent gradient summed over the batch and the gate gradient.
// One workgroup per head (1024 threads, four loads in flight each), fixed
// reduction order.
constexpr int kGateThreads = 1024;
//   dqf = sum_b dq;  dgate = sigma (1 - sigma) sum_{b,m,d} dq q_dyn
__global__ __launch_bounds__(kGateThreads) void bwd_gate_kernel(BwdGateParams a) {
  const int hd = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ float red[kGateThreads];
  const int MD = a.M * a.D;
#pragma unroll 4
  for (int md = tid; md < MD; md += kGateThreads) {
    float acc = 0.f;
    for (int b = 0; b < a.B; ++b) acc += a.dq[((int64_t)(b * a.H + hd) * a.M) * a.D + md];
    if (a.dqf) a.dqf[(int64_t)hd * MD + md] = acc;
  }
  if (!a.synthesis) return;
  float part = 0.f;
  for (int b = 0; b < a.B; ++b) {
    const int64_t base = ((int64_t)(b * a.H + hd) * a.M) * a.D;
#pragma unroll 4
    for (int md = tid; md < MD; md += kGateThreads) part += a.dq[base + md] * a.qd[base + md];
  }
  red[tid] = part;
  __syncthreads();
  for (int o = kGateThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0 && a.dgate) {
    const float sig = gate_sigma(a.gate[hd]);
    a.dgate[hd] = sig * (1.f - sig) * red[0];
  }
}

// Normalised latent gradient operand: workgroup (set, rb) finds the set's
// maximum (each of the set's workgroups reads it all, from L2) and writes
// the rows [16 rb, 16 rb + 16).
constexpr int kNormRows = 16;

__global__ __launch_bounds__(256) void bwd_norm_kernel(BwdNormParams a) {
  const int set = blockIdx.x;
  const int m0 = blockIdx.y * kNormRows;
  const int tid = threadIdx.x;
  const float alpha = a.gate ? gate_sigma(a.gate[set % a.H]) : 1.f;
  const float* src = a.src + (int64_t)set * a.M * a.D;
  const float* w = a.w + (int64_t)set * a.M * a.D;
  __shared__ float red[256];
  float mx = 0.f;
  const f32x4* src4 = reinterpret_cast<const f32x4*>(src);  // M D is a multiple of 4
#pragma unroll 4
  for (int i = tid; i < a.M * a.D / 4; i += 256) {
    const f32x4 v = src4[i];
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(alpha * v[0]), fabsf(alpha * v[1])),
                         fmaxf(fabsf(alpha * v[2]), fabsf(alpha * v[3]))));
  }
  red[tid] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  // rho = 2^k with max|g| <= rho < 2 max|g| (1 when g = 0)
  const int k = red[0] > 0.f ? (int)ceilf(log2f(red[0])) : 0;
  const float down = exp2f((float)-k);
  if (tid == 0 && blockIdx.y == 0) a.set_e[set] = (float)k - a.shift;
  const int wv = tid >> 6, d = tid & 63;
  for (int m = m0 + wv; m < min(a.M, m0 + kNormRows); m += 4) {  // one wave per latent row
    const bool live = d < a.D;
    const float g = live ? alpha * src[(int64_t)m * a.D + d] : 0.f;
    const float delta = wave_sum(g * (live ? w[(int64_t)m * a.D + d] : 0.f));
    if (live) st_op(a.rows, ((int64_t)set * a.Mpad + m) * a.D + d, a.dtype, g * down);
    if (d == 0) a.negd[(int64_t)set * a.M + m] = -delta * down;
  }
}

template <int MODE, typename T>
hipError_t lat_d(int D, const BwdLatParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 16: hipLaunchKernelGGL((bwd_lat_kernel<T, 16, MODE>), grid, dim3(64 * lat_waves<16>()), 0, s, p); break;
    case 32: hipLaunchKernelGGL((bwd_lat_kernel<T, 32, MODE>), grid, dim3(64 * lat_waves<32>()), 0, s, p); break;
    case 64: hipLaunchKernelGGL((bwd_lat_kernel<T, 64, MODE>), grid, dim3(64 * lat_waves<64>()), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t tok_lds(int M, int D) {
  const size_t Mk = (size_t)((M + 31) & ~31);
  return 3 * Mk * 2 * D + 3 * Mk * sizeof(float);
}

template <int MODE, typename T, int D>
hipError_t tok_launch(const BwdTokParams& p, hipStream_t s) {
  const size_t lds = tok_lds(p.M, D);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)bwd_tok_kernel<T, D, MODE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(p.B * p.H * p.wg_per_bh));
  hipLaunchKernelGGL((bwd_tok_kernel<T, D, MODE>), grid, dim3(64 * tok_waves<MODE, D>()), lds, s, p);
  return hipGetLastError();
}

template <int MODE, typename T>
hipError_t tok_d(int D, const BwdTokParams& p, hipStream_t s) {
  switch (D) {
    case 16: return tok_launch<MODE, T, 16>(p, s);
    case 32: return tok_launch<MODE, T, 32>(p, s);
    case 64: return tok_launch<MODE, T, 64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// The token pass sums over latents, so a head whose latents do not fit one
// workgroup's LDS runs as several launches over equal latent ranges (a
// multiple of 32 each), the later ones adding into the gradients the first
// one stored.
template <int MODE, typename T>
hipError_t tok_ranges(int D, const BwdTokParams& p, hipStream_t s) {
  const int nr = bwd_tok_latent_ranges(p.M, D);
  if (nr < 1) return hipErrorInvalidValue;
  if (nr == 1) return tok_d<MODE, T>(D, p, s);
  const int per = ((p.M + nr - 1) / nr + 31) & ~31;
  for (int m0 = 0; m0 < p.M; m0 += per) {
    BwdTokParams q = p;
    q.M = p.M - m0 < per ? p.M - m0 : per;
    q.lat_stat_stride = p.lat_stat_stride ? p.lat_stat_stride : p.M;
    q.lat_lse = p.lat_lse + m0;
    q.lat_negd = p.lat_negd + m0;
    for (int t = 0; t < 3; ++t)
      if (p.lat[t]) q.lat[t] = static_cast<const unsigned char*>(p.lat[t]) + (size_t)m0 * D * 2;
    q.accumulate = p.accumulate || m0 > 0;
    hipError_t e = tok_d<MODE, T>(D, q, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool bwd_lat_forms_delta2(int D) {
  return D == 16 ? lat_forms_delta2<16>() : D == 32 ? lat_forms_delta2<32>() : lat_forms_delta2<64>();
}
int bwd_latents_per_block(int D) { return 32 * (D <= 32 ? lat_waves<32>() : lat_waves<64>()); }
int bwd_tokens_per_tile() { return 32 * kBwdWaves; }
size_t bwd_tok_lds_bytes(int M, int D) { return tok_lds(M, D); }
int bwd_tok_latent_ranges(int M, int D) {
  for (int nr = 1; nr <= M; ++nr)
    if (tok_lds(((M + nr - 1) / nr + 31) & ~31, D) <= kBwdTokMaxLds) return nr;
  return 0;
}

hipError_t launch_bwd_lat(int dtype, int mode, int D, const BwdLatParams& p, hipStream_t s) {
  const int lpb = bwd_latents_per_block(D);
  const dim3 grid((unsigned)(p.B * p.H * p.nchunks), (unsigned)((p.M + lpb - 1) / lpb));
  if (dtype == kBF16) {
    if (mode == kBwdLatDec) return lat_d<kBwdLatDec, __bf16>(D, p, grid, s);
    if (mode == kBwdLatEnc) return lat_d<kBwdLatEnc, __bf16>(D, p, grid, s);
    return lat_d<kBwdLatSyn, __bf16>(D, p, grid, s);
  }
  if (mode == kBwdLatDec) return lat_d<kBwdLatDec, _Float16>(D, p, grid, s);
  if (mode == kBwdLatEnc) return lat_d<kBwdLatEnc, _Float16>(D, p, grid, s);
  return lat_d<kBwdLatSyn, _Float16>(D, p, grid, s);
}

hipError_t launch_bwd_tok(int dtype, int mode, int D, const BwdTokParams& p, hipStream_t s) {
  if (dtype == kBF16) {
    if (mode == kBwdTokFlare) return tok_ranges<kBwdTokFlare, __bf16>(D, p, s);
    return tok_ranges<kBwdTokSyn, __bf16>(D, p, s);
  }
  if (mode == kBwdTokFlare) return tok_ranges<kBwdTokFlare, _Float16>(D, p, s);
  return tok_ranges<kBwdTokSyn, _Float16>(D, p, s);
}


hipError_t launch_bwd_tok_prep(const BwdPrepParams& p, hipStream_t s) {
  const int64_t n = p.rows * (p.D / 8);
  hipLaunchKernelGGL(bwd_tok_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_bwd_rows(const BwdRowsParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.sets * p.Mpad * p.D;
  hipLaunchKernelGGL(bwd_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_bwd_dec_sums(const BwdSumsParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.sets * p.M * p.D * 4;
  hipLaunchKernelGGL(bwd_dec_sums_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_bwd_norm(const BwdNormParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_norm_kernel, dim3((unsigned)p.sets, (unsigned)((p.M + kNormRows - 1) / kNormRows)),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_bwd_add_sums(const BwdAddParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.sets * p.M * p.D * 4;
  hipLaunchKernelGGL(bwd_add_sums_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_bwd_gate(const BwdGateParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_gate_kernel, dim3((unsigned)p.H), dim3(kGateThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace flarepp
