// Decoder y = softmax_rows(scale k q^T) z: every token attends over the M
// latents (FLARE.py README, "FLARE++" listing, third attention call; "FLARE"
// listing, scatter step).
//
// The latents of one (batch, head) -- routing queries q as keys and encoded
// values z as values -- are loaded into LDS once per workgroup and stay
// resident while the workgroup walks its token tiles (persistent over
// tiles).  Tokens are the register side: each wave takes 32 * kNC tokens, loads
// their k rows from HBM into matrix-core operands (directly, or at D = 64
// through a per-wave LDS staging tile), sweeps the latents 32 at a time with
// the shared online-softmax tile, and writes its normalised y rows.  The value operand arrives with permuted rows so that
// each lane holds 4*NDB contiguous output columns of one token.
#include <type_traits>
#include <utility>

#include "flash_tile.hpp"
#include "kernels.hpp"

namespace flarepp {

namespace {

// 32-token column blocks per wave and waves per workgroup (build-time knobs)
#ifndef FLAREPP_DEC_NT_STORE
#define FLAREPP_DEC_NT_STORE 1
#endif
#ifndef FLAREPP_DEC_NC
#define FLAREPP_DEC_NC 1
#endif
constexpr int kNC = FLAREPP_DEC_NC;
// waves per workgroup (build-time knob for D <= 32)
#ifndef FLAREPP_DEC_WAVES
#define FLAREPP_DEC_WAVES 16
#endif
template <int D>
struct DecodeWaves {
  static constexpr int value = D >= 64 ? 8 : FLAREPP_DEC_WAVES;
};

constexpr int kMaxLdsBytes = 160 * 1024;

// f(integral_constant<K>) for K = 0, 1, ... in order while each returns true
template <int... K, typename F>
__device__ __forceinline__ bool all_slots(std::integer_sequence<int, K...>, F& f) {
  return (f(std::integral_constant<int, K>{}) && ...);
}

// LDS: the resident latents, then (STAGE) one staging tile per wave of its
// 32 * kNC token rows at pitch SP.  A staged wave reads and writes HBM one
// contiguous KiB per instruction and moves the rows into (and the outputs
// out of) the matrix-core layout through its staging tile; unstaged, each
// lane reads and writes 16-byte pieces of its own token's row, 32 rows per
// instruction.  At D = 64 a row is 128 bytes and the unstaged pattern holds
// the decoder well below the HBM rate of a plain copy; at D <= 32 the
// decoder is bound by its arithmetic and is not staged.
template <int D>
struct DecodeLds {
  static constexpr int DV = D < 32 ? 32 : D;
  static constexpr int KP = D + 8;  // latent row pitch (elements)
  static constexpr int SP = D + 8;  // staging row pitch (elements)
  static constexpr int kStageElems = DecodeWaves<D>::value * 32 * kNC * SP;
  static int zpitch(int Mk) { return Mk + 8; }
  static int elems(int Mk, bool stage) {
    return Mk * KP + DV * zpitch(Mk) + (stage ? kStageElems : 0);
  }
  // staged when the staging tiles fit beside the resident latents
  static bool stage(int Mk) { return D >= 64 && elems(Mk, true) * 2 <= kMaxLdsBytes; }
};

// A 16-byte store of the output y from the staging tile (a wave writes a
// contiguous KiB per instruction).  FLAREPP_DEC_NT_STORE: non-temporal, so y
// streams past the caches (nothing in the forward reads it again) and the
// next step's encoder does not pay for its write-back.  The unstaged path
// (32 or 64 bytes per token row, written by two lanes) keeps plain stores:
// non-temporal ones there left partial lines unmerged (16% more bytes
// written at D = 32) for no gain in time.
template <typename T>
__device__ __forceinline__ void y_store(T* p, u32x4 v) {
#if FLAREPP_DEC_NT_STORE
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
#else
  *reinterpret_cast<u32x4*>(p) = v;
#endif
}

// FIXUP = false: the decoder proper; a wave whose sums leave the fixed
// reference's range records that tile (its stores still go out and are
// overwritten later).
// FIXUP = true: the same workgroups again, recomputing only the recorded
// tiles by the exact two-pass method (a workgroup with none exits at once).
// The split keeps the rare exact path's registers out of the main kernel.
// LSE: also store each token's log2 row sum plus reference (training).
// STAGE: token rows and outputs pass through a per-wave LDS staging tile.
template <typename T, int D, bool FIXUP, bool LSE, bool STAGE>
__global__ __launch_bounds__(64 * DecodeWaves<D>::value) void
decode_kernel(DecodeParams a) {
  constexpr int kNW = DecodeWaves<D>::value;
  constexpr int kTokTile = 32 * kNC * kNW;
  using Tile = FlashTile<T, D, kNC>;
  using V8 = typename Tile::V8;
  constexpr int KD = Tile::KD, DV = Tile::DV, NDB = Tile::NDB;
  constexpr int KP = DecodeLds<D>::KP;
  constexpr int SP = DecodeLds<D>::SP;
  static_assert(!STAGE || D >= 16, "staging moves whole 16-byte pieces of rows");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  T* qs = reinterpret_cast<T*>(lds_raw);

  const int Mk = (a.M + 31) & ~31;
  const int ZP = Mk + 8;
  T* zs = qs + Mk * KP;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int bh = blockIdx.x / a.wg_per_bh;
  const int part = blockIdx.x - bh * a.wg_per_bh;
  const int b = bh / a.H, hd = bh - b * a.H;
  // this wave's staging tile (STAGE): rows cb * 32 + j, pitch SP
  T* sg = zs + DV * ZP + wave * (32 * kNC * SP);
  // staged HBM access: instruction i of a 32-row block moves its bytes
  // [1024 i, 1024 i + 1024); lane l's 16 bytes are row i * kRPI + l / kCPR,
  // elements 8 (l % kCPR) .. +7
  constexpr int kCPR = D / 8, kRPI = 64 / kCPR;
  const int srow = lane / kCPR, scol = 8 * (lane % kCPR);

  // this wave's record: bit i = the workgroup's i-th tile (i < 64), and
  // 1 + the first ordinal >= 64 from which every tile is recomputed (0: none)
  unsigned long long* rec = a.redo + ((int64_t)blockIdx.x * kNW + wave) * 2;
  uint64_t fx_bad = 0;
  int64_t fx_from = -1;
  if constexpr (FIXUP) {
    fx_bad = rec[0];
    fx_from = (int64_t)rec[1] - 1;
    if (!__syncthreads_or(fx_bad != 0 || fx_from >= 0)) return;  // workgroup-uniform
  }

  // resident latents: q rows [0, Mk) and the value operand rows [0, DV);
  // the largest |z| of the head is taken on the way (it bounds every
  // accumulator, which makes the overflow test per tile a row-sum test)
  __shared__ unsigned zmax_bits;
  if (tid == 0) zmax_bits = 0u;
  __syncthreads();
  {
    const T* qg = reinterpret_cast<const T*>(a.q) + b * a.q_b_stride + hd * a.q_h_stride;
    constexpr int G8 = D / 8;
    const bool raw = a.qscale > 0.f;  // caller latents [.., M, D]: scale, zero rows >= M
    for (int u = tid; u < Mk * G8; u += 64 * kNW) {
      const int row = u / G8, e = u - row * G8;
      u32x4 w;
      if (!raw) w = ldg16(qg + (int64_t)row * D + 8 * e);
      else if (row < a.M) w = scaled8<T>(qg + (int64_t)row * D + 8 * e, a.qscale);
      else w = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&qs[row * KP + 8 * e]) = w;
    }
    // z arrives in natural [m][d] rows; the value operand in LDS is z^T with
    // rows d permuted (value_row) and latents in key-slot order, rows
    // D <= d < DV zero
    const T* zg = reinterpret_cast<const T*>(a.zt) + (int64_t)bh * a.Mpad * D;
    unsigned zb = 0u;  // max over this thread's values of |z| as ordered bits
    for (int u = tid; u < Mk * G8; u += 64 * kNW) {
      const int m = u / G8, e = u - m * G8;
      const u32x4 v = ldg16(zg + (int64_t)m * D + 8 * e);
      const int col = (m & ~31) + key_slot(m & 31);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const unsigned short bits = (unsigned short)(v[j >> 1] >> (16 * (j & 1)));
        const int d = 8 * e + j;
        zs[((d & ~31) + value_row(d & 31)) * ZP + col] = __builtin_bit_cast(T, bits);
        zb = max(zb, __float_as_uint(fabsf((float)__builtin_bit_cast(T, bits))));
      }
    }
    if constexpr (D < DV) {
      for (int u = tid; u < (DV - D) * Mk; u += 64 * kNW) {
        const int d = D + u / Mk, c = u - (u / Mk) * Mk;
        zs[value_row(d) * ZP + c] = (T)0.f;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) zb = max(zb, (unsigned)__shfl_xor((int)zb, o));
    if (lane == 0) atomicMax(&zmax_bits, zb);
  }
  __syncthreads();
  const float zmax = __uint_as_float(zmax_bits);  // NaN bits order above infinity

  const T* kg = reinterpret_cast<const T*>(a.k) + (int64_t)bh * a.N * D;
  T* yg = reinterpret_cast<T*>(a.y) + (int64_t)bh * a.N * D;
  const int64_t ntiles = (a.N + kTokTile - 1) / kTokTile;
  const int nfull = a.M / 32, mtail = a.M - 32 * nfull;

  // lane-constant byte offsets of the resident operands; a latent group G
  // adds G * (32 rows) to the key operand and G * (32 slots) to the values
  int kl[KD];
#pragma unroll
  for (int kd = 0; kd < KD; ++kd) kl[kd] = (r * KP + 16 * kd + 8 * h) * (int)sizeof(T);
  int vl[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) vl[db] = ((32 * db + r) * ZP + 8 * h) * (int)sizeof(T);
  const unsigned char* qsb = reinterpret_cast<const unsigned char*>(qs);
  const unsigned char* zsb = reinterpret_cast<const unsigned char*>(zs);
  constexpr int KSTEP = 32 * KP * (int)sizeof(T);  // bytes per latent group, key operand
  constexpr int VSTEP = 32 * (int)sizeof(T);       // bytes per latent group, value operand
  auto kop_at = [&](int G, V8 (&kop)[KD]) {
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      if (16 * kd + 8 * h < D)
        kop[kd] = *reinterpret_cast<const V8*>(qsb + kl[kd] + G * KSTEP);
      else
        kop[kd] = bitcast_u4<V8>(u32x4{0u, 0u, 0u, 0u});
    }
  };
  auto vop_at = [&](int G, V8 (&vop)[NDB][2]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        vop[db][kk] =
            *reinterpret_cast<const V8*>(zsb + vl[db] + G * VSTEP + kk * 16 * (int)sizeof(T));
  };

  // token rows of one tile for this wave: unstaged, already the
  // register-side operand; staged, the rows as they lie in HBM (to_operand
  // rearranges them).  Rows past N re-read row N-1 (every token column is
  // independent, and such a column's outputs equal row N-1's), so the loads
  // carry no condition and the compiler can wait for exactly the loads a
  // tile needs.
  auto load_tokens = [&](int64_t tile, V8 (&dst)[kNC][KD]) {
    const int64_t nb = tile * kTokTile + wave * 32 * kNC;
    if constexpr (STAGE) {
#pragma unroll
      for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
        for (int i = 0; i < KD; ++i) {
          const int64_t n = min(nb + cb * 32 + i * kRPI + srow, a.N - 1);
          dst[cb][i] = bitcast_u4<V8>(ldg16(kg + n * D + scol));
        }
      return;
    }
#pragma unroll
    for (int cb = 0; cb < kNC; ++cb) {
      const int64_t n = min(nb + cb * 32 + r, a.N - 1);
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) {
        const int d0 = 16 * kd + 8 * h;
        if constexpr (D >= 16) {
          dst[cb][kd] = bitcast_u4<V8>(ldg16(kg + n * D + d0));
        } else {  // D = 8: the upper half of the K=16 step is zero padding
          if (d0 < D) dst[cb][kd] = bitcast_u4<V8>(ldg16(kg + n * D + d0));
          else dst[cb][kd] = bitcast_u4<V8>(u32x4{0u, 0u, 0u, 0u});
        }
      }
    }
  };

  // register-side operand of a tile from what load_tokens fetched
  auto to_operand = [&](const V8 (&src)[kNC][KD], V8 (&q)[kNC][KD]) {
    if constexpr (STAGE) {
#pragma unroll
      for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
        for (int i = 0; i < KD; ++i)
          *reinterpret_cast<V8*>(sg + (cb * 32 + i * kRPI + srow) * SP + scol) = src[cb][i];
#pragma unroll
      for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
        for (int kd = 0; kd < KD; ++kd)
          q[cb][kd] = *reinterpret_cast<const V8*>(sg + (cb * 32 + r) * SP + 16 * kd + 8 * h);
    } else {
#pragma unroll
      for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) q[cb][kd] = src[cb][kd];
    }
  };

// y = O / l; lane (h, r) owns columns 32db + 16h .. +15 of token r (staged:
// they go to the staging tile and leave it a contiguous KiB per store).
// Every lane stores, so the number of stores per tile is fixed and the
// waits before a tile count only its own loads (a conditional store would
// make the compiler also wait for the previous tile's stores).  A column
// past N holds row N-1's inputs and so exactly row N-1's results: it
// stores them to row N-1 again.
auto store_tile = [&](int64_t nb, const auto& t) {
#pragma unroll
    for (int cb = 0; cb < kNC; ++cb) {
      const float l = t.row_sum(cb);
      const float inv = 1.0f / l;
      const int64_t n = min(nb + cb * 32 + r, a.N - 1);
      if constexpr (LSE)  // both halves of the wave hold token r's sum
        a.lse_out[(int64_t)bh * a.N + n] = log2f(l) + t.reference(cb);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d0 = 32 * db + 16 * h;
        if (d0 < D) {  // lane-dependent only for D < 32
          T out[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) out[v] = (T)(t.o[db][cb][v] * inv);
          T* dst = STAGE ? sg + (cb * 32 + r) * SP + d0 : yg + n * D + d0;
          if constexpr (D >= 16) {
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&out[0]);
            *reinterpret_cast<u32x4*>(dst + 8) = *reinterpret_cast<const u32x4*>(&out[8]);
          } else {
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&out[0]);
          }
        }
      }
      if constexpr (STAGE) {
#pragma unroll
        for (int i = 0; i < KD; ++i) {
          const int row = i * kRPI + srow;
          const u32x4 v = *reinterpret_cast<const u32x4*>(sg + (cb * 32 + row) * SP + scol);
          y_store(yg + min(nb + cb * 32 + row, a.N - 1) * D + scol, v);
        }
      }
    }
  };

  // One tile: the wave's 32 * kNC token rows arrive as qop (register
  // operand); sweep all latents and store y.  Returns true when the fixed
  // reference failed: what was stored is then wrong and the fix-up pass
  // recomputes the tile.  A wave whose rows all lie past N (last tile of a
  // ragged N) computes row N-1 and stores it again, which keeps the store
  // count free of branches.
  auto process_tile = [&](int64_t tile, const V8 (&qop)[kNC][KD])
                          __attribute__((always_inline)) -> bool {
    const int64_t nb = tile * kTokTile + wave * 32 * kNC;
    Tile st;
    st.reset();
    to_operand(qop, st.q);
    // latent groups of 32: group 0, then full groups as a two-stage
    // pipeline (the score product of group G+1 is issued before the
    // softmax of group G, two score buffers alternating), then a masked
    // tail group
    f32x16 sa[kNC], sb[kNC];
    {
      V8 kop[KD];
      kop_at(0, kop);
      st.scores(kop, sa);
      V8 vop[NDB][2];
      vop_at(0, vop);
      if (nfull > 0) st.template first<false>(sa, vop, 32, h);
      else st.template first<true>(sa, vop, mtail, h);
    }
    if (nfull > 1) {
      {
        V8 kop[KD];
        kop_at(1, kop);
        st.scores(kop, sa);
      }
      int G = 1;
      for (; G + 2 < nfull; G += 2) {  // groups G and G+1, then G+2's scores
        {
          V8 kop[KD];
          kop_at(G + 1, kop);
          st.scores(kop, sb);
          V8 vop[NDB][2];
          vop_at(G, vop);
          st.template next<false>(sa, vop, 32, h);
        }
        V8 kop[KD];
        kop_at(G + 2, kop);
        st.scores(kop, sa);
        V8 vop[NDB][2];
        vop_at(G + 1, vop);
        st.template next<false>(sb, vop, 32, h);
      }
      if (G + 1 < nfull) {  // two full groups left
        V8 kop[KD];
        kop_at(G + 1, kop);
        st.scores(kop, sb);
        V8 vop[NDB][2];
        vop_at(G, vop);
        st.template next<false>(sa, vop, 32, h);
        vop_at(G + 1, vop);
        st.template next<false>(sb, vop, 32, h);
      } else {  // one
        V8 vop[NDB][2];
        vop_at(G, vop);
        st.template next<false>(sa, vop, 32, h);
      }
    }
    if (nfull > 0 && mtail > 0) {
      V8 kop[KD];
      kop_at(nfull, kop);
      st.scores(kop, sa);
      V8 vop[NDB][2];
      vop_at(nfull, vop);
      st.template next<true>(sa, vop, mtail, h);
    }
    const bool bad = st.overflowed_bounded(zmax);  // recomputed exactly in the fix-up pass
    store_tile(nb, st);
    return bad;
  };

  // Sums out of range for the fixed reference: exact two-pass recompute of
  // this wave's tokens of one tile (true maxima over all latents first, then
  // the sums).  Kept out of the main loop so that its registers are not live
  // beside the prefetched token rows.
  auto exact_tile = [&](int64_t tile, const V8 (&qop)[kNC][KD]) {
    const int64_t nb = tile * kTokTile + wave * 32 * kNC;
    using Exact = FlashTile<T, D, kNC, true>;
    Exact ex;
    ex.reset();
    to_operand(qop, ex.q);
    const int ngrp = nfull + (mtail > 0 ? 1 : 0);
    f32x16 sa[kNC];
    float mx[kNC];
#pragma unroll
    for (int cb = 0; cb < kNC; ++cb) mx[cb] = -__builtin_inff();
    for (int G = 0; G < ngrp; ++G) {
      V8 kop[KD];
      kop_at(G, kop);
      ex.scores(kop, sa);
      Exact::mask(sa, a.M - 32 * G, h);
      float gm[kNC];
      Exact::colmax(sa, gm);
#pragma unroll
      for (int cb = 0; cb < kNC; ++cb) mx[cb] = fmaxf(mx[cb], gm[cb]);
    }
    ex.set_reference(sa, mx);
    for (int G = 0; G < ngrp; ++G) {
      V8 kop[KD];
      kop_at(G, kop);
      ex.scores(kop, sa);
      V8 vop[NDB][2];
      vop_at(G, vop);
      ex.template next<true>(sa, vop, a.M - 32 * G, h);
    }
    store_tile(nb, ex);
  };

  // The workgroup walks tiles part, part + wg_per_bh, ...; the token rows of
  // the next kDepth - 1 tiles are in flight in a ring of register sets while
  // the current tile is computed (the loop is unrolled by kDepth so the sets
  // never need copying).  Two tiles in flight measured no faster than one.
  constexpr int kDepth = 2;
  V8 ring[kDepth][kNC][KD];
  if constexpr (!FIXUP) {
    // Tiles that overflowed are remembered by their ordinal i among this
    // workgroup's tiles (bit i of a mask for i < 64; past that, every tile
    // from the first such ordinal on).
    uint64_t bad = 0;
    int64_t bad_from = -1;
    auto note_bad = [&](int64_t i) {
      if (i < 64) bad |= (uint64_t)1 << i;
      else if (bad_from < 0) bad_from = i;
    };
    const int64_t step = a.wg_per_bh;
    int64_t tile = part, ord = 0;
    // Prologue: the first kDepth - 1 ring slots, each load followed by as
    // many store instructions as a tile issues (single bytes to distinct
    // places of this wave's record, which is written in full after the
    // loop).  The loop is then entered with the same memory-counter history
    // as from its back edge, and the compiler's wait before every tile
    // counts only that tile's loads, never the stores of the tiles before.
    constexpr int kTileStores = kNC * ((STAGE ? KD : NDB * (D >= 16 ? 2 : 1)) + (LSE ? 1 : 0));
    static_assert(2 * kTileStores <= 16, "record too small for the prologue stores");
    unsigned char* pad = reinterpret_cast<unsigned char*>(rec);
#pragma unroll
    for (int k = 0; k + 1 < kDepth; ++k) {
      load_tokens(tile + k * step, ring[k]);
#pragma unroll
      for (int j = 0; j < kTileStores; ++j) pad[2 * j] = (unsigned char)k;
    }
    // one tile on ring slot K; false once the walk is over.  The loop below
    // has a single exit, so its header is reached only from the prologue and
    // from its back edge.
    auto slot = [&](auto kc) __attribute__((always_inline)) -> bool {
      constexpr int K = decltype(kc)::value;
      if (tile >= ntiles) return false;
      // issued even past the last tile (rows clamp to N-1, results unused)
      load_tokens(tile + (kDepth - 1) * step, ring[(K + kDepth - 1) % kDepth]);
      if (process_tile(tile, ring[K])) note_bad(ord);
      tile += step;
      ++ord;
      return true;
    };
    while (all_slots(std::make_integer_sequence<int, kDepth>{}, slot)) {
    }
    if (lane == 0) {  // written for every wave, so no clearing is needed
      rec[0] = bad;
      rec[1] = (unsigned long long)(bad_from + 1);
    }
  } else {
    int64_t ord = 0;
    for (int64_t t = part; t < ntiles; t += a.wg_per_bh, ++ord) {
      const bool redo =
          ord < 64 ? ((fx_bad >> ord) & 1) != 0 : (fx_from >= 0 && ord >= fx_from);
      if (!redo) continue;
      load_tokens(t, ring[0]);
      exact_tile(t, ring[0]);
    }
  }
}

// fp32 path: one thread per token, latents streamed through LDS 32 at a time.
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeParams a) {
  constexpr int TM = 32;
  __shared__ float qsm[TM][D];
  __shared__ float zsm[TM][D];
  const int tid = threadIdx.x;
  // one-dimensional grid of ceil(N / 256) blocks per (b, h), heads outermost
  const int64_t bpb = (a.N + 255) / 256;
  const int bh = (int)(blockIdx.x / bpb);
  const int b = bh / a.H, h = bh - b * a.H;
  const int64_t n = ((int64_t)blockIdx.x - (int64_t)bh * bpb) * 256 + tid;
  const bool valid = n < a.N;
  const float* kb = reinterpret_cast<const float*>(a.k) + (int64_t)bh * a.N * D;
  const float* qb = reinterpret_cast<const float*>(a.q) + b * a.q_b_stride + h * a.q_h_stride;
  const float* zb = reinterpret_cast<const float*>(a.zt) + (int64_t)bh * a.Mpad * D;
  float kr[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kr[d] = valid ? kb[n * D + d] : 0.f;
    o[d] = 0.f;
  }
  float mref = -__builtin_inff(), l = 0.f;
  for (int mb = 0; mb < a.M; mb += TM) {
    const int tv = min(TM, a.M - mb);
    for (int e = tid; e < TM * D; e += blockDim.x) {
      const int j = e / D, d = e - j * D;
      const float qv = j < tv ? qb[(int64_t)(mb + j) * D + d] : 0.f;
      qsm[j][d] = a.qscale > 0.f ? a.qscale * qv : qv;
      zsm[j][d] = j < tv ? zb[(int64_t)(mb + j) * D + d] : 0.f;
    }
    __syncthreads();
    float s[TM];
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(kr[d], qsm[j][d], acc);
      s[j] = j < tv ? acc : -__builtin_inff();
      mx = fmaxf(mx, s[j]);
    }
    if (mx > mref) {
      const float sc = exp2f(mref - mx);
      l *= sc;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= sc;
      mref = mx;
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const float p = exp2f(s[j] - mref);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, zsm[j][d], o[d]);
    }
    __syncthreads();
  }
  if (valid) {
    float* yb = reinterpret_cast<float*>(a.y) + (int64_t)bh * a.N * D;
    const float inv = 1.0f / l;
    if (a.lse_out) a.lse_out[(int64_t)bh * a.N + n] = mref + log2f(l);
#pragma unroll
    for (int d = 0; d < D; ++d) yb[n * D + d] = o[d] * inv;
  }
}

template <typename T, int D, bool LSE, bool STAGE>
hipError_t launch_mfma_s(const DecodeParams& p, hipStream_t s) {
  const int Mk = (p.M + 31) & ~31;
  const size_t lds = (size_t)DecodeLds<D>::elems(Mk, STAGE) * sizeof(T);
  if (lds > 64 * 1024) {
    for (const void* f : {(const void*)decode_kernel<T, D, false, LSE, STAGE>,
                          (const void*)decode_kernel<T, D, true, LSE, STAGE>}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
  }
  const dim3 grid((unsigned)(p.B * p.H * p.wg_per_bh)), block(64 * DecodeWaves<D>::value);
  hipLaunchKernelGGL((decode_kernel<T, D, false, LSE, STAGE>), grid, block, lds, s, p);
  hipLaunchKernelGGL((decode_kernel<T, D, true, LSE, STAGE>), grid, block, lds, s, p);
  return hipGetLastError();
}

template <typename T, int D, bool LSE>
hipError_t launch_mfma(const DecodeParams& p, hipStream_t s) {
  if constexpr (D >= 64) {
    if (DecodeLds<D>::stage((p.M + 31) & ~31)) return launch_mfma_s<T, D, LSE, true>(p, s);
  }
  return launch_mfma_s<T, D, LSE, false>(p, s);
}

template <typename T, bool LSE>
hipError_t launch_mfma_d(int D, const DecodeParams& p, hipStream_t s) {
  switch (D) {
    case 8: return launch_mfma<T, 8, LSE>(p, s);
    case 16: return launch_mfma<T, 16, LSE>(p, s);
    case 32: return launch_mfma<T, 32, LSE>(p, s);
    case 64: return launch_mfma<T, 64, LSE>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_f32(const DecodeParams& p, hipStream_t s) {
  const int64_t blocks = (p.N + 255) / 256 * p.B * p.H;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  hipLaunchKernelGGL((decode_f32_kernel<D>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int decode_waves(int D) { return D >= 64 ? DecodeWaves<64>::value : DecodeWaves<32>::value; }

int decode_tokens_per_tile(int D) {
  return 32 * kNC * (D >= 64 ? DecodeWaves<64>::value : DecodeWaves<32>::value);
}

int decode_lds_bytes(int M, int D, int dtype) {
  if (dtype == kF32) return 0;
  const int Mk = (M + 31) & ~31;
  switch (D) {
    case 8: return DecodeLds<8>::elems(Mk, false) * 2;
    case 16: return DecodeLds<16>::elems(Mk, false) * 2;
    case 32: return DecodeLds<32>::elems(Mk, false) * 2;
    case 64: return DecodeLds<64>::elems(Mk, DecodeLds<64>::stage(Mk)) * 2;
    default: return -1;
  }
}

hipError_t launch_decode(int dtype, int D, const DecodeParams& p, hipStream_t s) {
  const bool lse = p.lse_out != nullptr;
  if (dtype == kBF16)
    return lse ? launch_mfma_d<__bf16, true>(D, p, s) : launch_mfma_d<__bf16, false>(D, p, s);
  if (dtype == kF16)
    return lse ? launch_mfma_d<_Float16, true>(D, p, s) : launch_mfma_d<_Float16, false>(D, p, s);
  switch (D) {
    case 8: return launch_f32<8>(p, s);
    case 16: return launch_f32<16>(p, s);
    case 32: return launch_f32<32>(p, s);
    case 64: return launch_f32<64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace flarepp
