// Split-N encoder: per token chunk, the online-softmax partials of
//   z = softmax_rows(scale q k^T) v        (encode, FLARE.py README "FLARE++")
//   q_dyn = softmax_rows(scale q0 k0^T) k0 (synthesis, keys = values = k0)
// as (reference m, row sum l, unnormalised output O) per latent row, which
// the combine kernel merges with log-sum-exp weights (issue #2024,
// "Multi-GPU context parallelism": exact token-sharded encoder).
//
// One workgroup = one (batch, head, token chunk).  Its waves split the
// latents (32 * kNC per wave); every wave consumes the same K/V tiles, which
// are staged in LDS in their natural [token][d] layout.  The P.V product contracts over tokens, so
// its matrix-core operand needs V with tokens along k: it is read with the
// transposing LDS load (ds_read_b64_tr_b16) instead of being transposed in
// flight.  Tiles of kTJ tokens rotate over three LDS buffers; the loads of
// tile t+1 are in flight while tile t is computed.
#include "flash_tile.hpp"
#include "kernels.hpp"

namespace flarepp {

namespace {

// 32-column blocks per wave (build-time knob; 1 keeps the register
// footprint low enough for four waves per SIMD)
#ifndef FLAREPP_ENC_NC
#define FLAREPP_ENC_NC 1
#endif
constexpr int kNC = FLAREPP_ENC_NC;
constexpr int kMaxWaves = 16 / kNC;   // waves per workgroup for M = 512
#ifndef FLAREPP_ENC_TILE
#define FLAREPP_ENC_TILE 128
#endif
constexpr int kTJ = FLAREPP_ENC_TILE;  // tokens per LDS tile (chunk granularity)
// Tiles of 64 tokens at D = 64: with 128 the unrolled tile body held 268
// VGPRs and two staged tensors took 96 KB of LDS -- one 4-wave workgroup,
// one wave per SIMD; with 64 it fits 204 VGPRs and 48 KB, two waves per
// SIMD (measured -20% for the encoder at B8 H16 N16384 M128 D64 fp16).
template <int D>
constexpr int kTileTokens = D >= 64 ? 64 : kTJ;
// Waves per SIMD the registers must allow.  An 8-wave bf16 workgroup at
// D <= 32 (M = 129..256) is held to 128 VGPRs, without spills, so that two
// workgroups share a CU (it took 154, one per CU): same-box A/B at
// B2 H8 N40000 M256 D32, synthesis 37.7 -> 33.3 us, encode unchanged; at
// D = 16 the encode 31.7 -> 28.6 us.  fp16 would spill there and keeps 1.
template <typename T, int D, int NW>
constexpr int kMinWaves = D >= 64 ? 2 : (D <= 32 && NW == 8 && std::is_same<T, __bf16>::value) ? 4 : 1;
// LDS tiles rotate over three buffers: with the score product running one
// group ahead, a wave may still read tile t-1 while others fill tile t+1.
constexpr int kNBUF = 3;

// LDS tile layout: token rows of 2*D bytes in natural [token][d] order, the
// 16-byte chunks of row `row` XOR-permuted by swz(row) so that both the
// K-operand reads (16 rows x 16 bytes per phase) and the transposing V reads
// hit distinct banks.
template <int D>
struct TileLayout {
  static constexpr int ROWB = 2 * D;           // bytes per token row
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPB = 256 / ROWB;       // rows per 256 bytes (all banks)
  static constexpr int TILEB = kTileTokens<D> * ROWB;  // bytes per tile per tensor
  __device__ __forceinline__ static int swz(int row) { return (row / RPB) % CPR; }
  __device__ __forceinline__ static int offset(int row, int byte) {  // byte within row
    return row * ROWB + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
  }
};

template <typename T, int D, int NW, bool SHARED_KV>
__global__ __launch_bounds__(64 * NW, (kMinWaves<T, D, NW>)) void encode_split_kernel(EncodeParams a) {
  constexpr int kTJ = kTileTokens<D>;  // tokens per LDS tile
  constexpr int kGPT = kTJ / 32;       // 32-key groups per tile
  using Tile = FlashTile<T, D, kNC>;
  using V8 = typename Tile::V8;
  using L = TileLayout<D>;
  constexpr int KD = Tile::KD, NDB = Tile::NDB;
  constexpr int NTEN = SHARED_KV ? 1 : 2;               // tensors staged per tile
  constexpr int LOADS = L::TILEB / 1024;                // 1 KB wave loads per tensor
  static_assert(L::TILEB % 1024 == 0, "tile must be a whole number of wave loads");

  // Three tile buffers as three distinct LDS objects: reads from one buffer
  // then provably do not alias the direct loads landing in another, so the
  // compiler does not make them wait for those loads.
  __shared__ __attribute__((aligned(16))) unsigned char lds0[NTEN * L::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[NTEN * L::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char lds2[NTEN * L::TILEB];
  auto buf_c = [&](auto bc) -> unsigned char* {
    constexpr int B = decltype(bc)::value;
    if constexpr (B == 0) return lds0;
    else if constexpr (B == 1) return lds1;
    else return lds2;
  };
  auto buf_rt = [&](int b) -> unsigned char* { return b == 0 ? lds0 : b == 1 ? lds1 : lds2; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int bh = blockIdx.x / a.nchunks;
  const int chunk = blockIdx.x - bh * a.nchunks;
  const int b = bh / a.H, hd = bh - b * a.H;
  const int lat0 = (int)blockIdx.y * (NW * 32 * kNC);  // first latent of this workgroup

  if (a.gate != nullptr && gate_sigma(a.gate[hd]) == 0.f) return;  // closed gate: no synthesis

  const int64_t n0 = (int64_t)chunk * a.chunk_tokens;
  const int64_t n1 = min(a.N, n0 + a.chunk_tokens);
  const int ntok = (int)(n1 - n0);
  const int ntiles = (ntok + kTJ - 1) / kTJ;
  const T* kbase = reinterpret_cast<const T*>(a.k) + (int64_t)bh * a.N * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (int64_t)bh * a.N * D;

  Tile st;
  st.reset();
  {
    const T* qb = reinterpret_cast<const T*>(a.q) + b * a.q_b_stride + hd * a.q_h_stride;
    const int col = lat0 + wave * 32 * kNC + r;
    const bool raw = a.qscale > 0.f;  // caller latents [.., M, D]: scale, zero rows >= M
#pragma unroll
    for (int cb = 0; cb < kNC; ++cb) {
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) {
        const int d0 = 16 * kd + 8 * h, row = col + 32 * cb;
        if (d0 >= D || (raw && row >= a.M))
          st.q[cb][kd] = bitcast_u4<V8>(u32x4{0u, 0u, 0u, 0u});
        else if (raw)
          st.q[cb][kd] = bitcast_u4<V8>(scaled8<T>(qb + (int64_t)row * D + d0, a.qscale));
        else
          st.q[cb][kd] = bitcast_u4<V8>(ldg16(qb + (int64_t)row * D + d0));
      }
    }
  }

  // HBM -> LDS with no registers: a wave load moves 1 KB, lane i's 16 bytes
  // landing at byte 16*i of it.  Rows past the chunk end re-read the chunk's
  // last token (finite data; those keys are masked to probability 0).
  auto issue_loads = [&](unsigned char* dst, int t) {
    const int lim = ntok - 1 - t * kTJ;  // last valid row of the tile
    const T* kt = kbase + (n0 + (int64_t)t * kTJ) * D;
    const T* vt = vbase + (n0 + (int64_t)t * kTJ) * D;
    for (int ld = wave; ld < NTEN * LOADS; ld += NW) {
      const int ten = ld / LOADS, li = ld - ten * LOADS;
      const int o = li * 1024 + 16 * lane;
      const int row = o / L::ROWB;
      const int clog = ((o % L::ROWB) >> 4) ^ L::swz(row);
      const int eoff = min(row, lim) * D + 8 * clog;
      // the values are read only here; the keys are read again by the decoder
      if (ten == 0) global_to_lds16(kt + eoff, dst + li * 1024);
      else global_to_lds16_nt(vt + eoff, dst + ten * L::TILEB + li * 1024);
    }
  };
  // Entering tile t (buffer B = t % 3): its loads, issued one tile earlier,
  // are complete in every wave after the barrier, which also retires all
  // reads of tile t-2 -- whose buffer then receives tile t+1.
  auto enter_tile = [&](auto bc, int t) {
    constexpr int B = decltype(bc)::value;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) issue_loads(buf_c(IntC<(B + 1) % kNBUF>{}), t + 1);
  };

  // Lane-constant parts of the LDS operand addresses.  The swizzle of a row
  // only depends on the row's position within its 32-key group, so a group
  // adds an immediate.
  int kaddr[KD];
#pragma unroll
  for (int kd = 0; kd < KD; ++kd) kaddr[kd] = L::offset(r, 2 * (16 * kd + 8 * h));
  // V^T operand through the transposing LDS read: in each 16-lane group,
  // source lane 4k+q addresses key k, columns d0+4q..d0+4q+3, and lane j
  // receives column d0+j of keys 0..3.
  const int tr_k = (lane & 15) >> 2, tr_q = lane & 3;
  int vaddr[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * tr_q;
    if (d >= D) d = 0;  // feeds only padded output rows
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
      vaddr[db][aa] = (NTEN - 1) * L::TILEB + L::offset(8 * aa + 4 * h + tr_k, 2 * d);
  }
  auto kop_at = [&](const unsigned char* base, int grp, V8 (&kop)[KD]) {
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      if (16 * kd < D && (D >= 16 || h == 0))
        kop[kd] = *reinterpret_cast<const V8*>(base + kaddr[kd] + grp * 32 * L::ROWB);
      else
        kop[kd] = bitcast_u4<V8>(u32x4{0u, 0u, 0u, 0u});
    }
  };
  auto vop_at = [&](const unsigned char* base, int grp, V8 (&vop)[NDB][2]) {
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
        vop[db][kk] = __builtin_bit_cast(V8, short8v{part[0][0], part[0][1], part[0][2], part[0][3],
                                                     part[1][0], part[1][1], part[1][2], part[1][3]});
      }
  };

  // Key groups of 32 tokens, kGPT per tile.  Tile 0 runs plainly (its first
  // group sets the references).  Full tiles 1 .. nft-1 run as a two-stage
  // pipeline -- the score product of the next group is issued before the
  // softmax of the current one, two score buffers alternating (group g of a
  // tile in sa for even g, sb for odd g) -- with the buffer rotation unrolled
  // so every LDS address is a lane base plus an immediate.  A partial last
  // tile follows.
  static_assert(kGPT % 2 == 0, "tiles hold an even number of key groups");
  const int nft = ntok / kTJ;  // full tiles
  f32x16 sa[kNC], sb[kNC];
  auto sbuf = [&](auto gc) -> f32x16(&)[kNC] {
    if constexpr (decltype(gc)::value % 2 == 0) return sa;
    else return sb;
  };
  issue_loads(lds0, 0);
  enter_tile(IntC<0>{}, 0);
  static_for<kGPT>([&](auto gc) {
    constexpr int g = decltype(gc)::value;
    if (32 * g < ntok) {
      const int kvalid = min(32, ntok - 32 * g);
      V8 kop[KD];
      kop_at(lds0, g, kop);
      st.scores(kop, sa);
      V8 vop[NDB][2];
      vop_at(lds0, g, vop);
      if constexpr (g == 0) {
        if (kvalid == 32) st.template first<false>(sa, vop, 32, h);
        else st.template first<true>(sa, vop, kvalid, h);
      } else {
        if (kvalid == 32) st.template next<false>(sa, vop, 32, h);
        else st.template next<true>(sa, vop, kvalid, h);
      }
    }
  });
  // groups 0 .. kGPT-2 of a full tile in `cur`: on entry sbuf(0) holds the
  // scores of group 0, on exit sbuf(kGPT-1) those of the last group
  auto tile_groups = [&](const unsigned char* cur) {
    static_for<kGPT - 1>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      V8 kop[KD];
      kop_at(cur, g + 1, kop);
      st.scores(kop, sbuf(IntC<g + 1>{}));
      V8 vop[NDB][2];
      vop_at(cur, g, vop);
      st.template next<false>(sbuf(gc), vop, 32, h);
    });
  };
  // tile t in buffer B whose successor t+1 is also full; on entry sa holds
  // the scores of tile t's first group, on exit those of tile t+1's
  auto tile_body = [&](auto bc, int t) {
    constexpr int B = decltype(bc)::value, BN = (B + 1) % kNBUF;
    const unsigned char* cur = buf_c(bc);
    tile_groups(cur);
    enter_tile(IntC<BN>{}, t + 1);
    V8 kop[KD];
    kop_at(buf_c(IntC<BN>{}), 0, kop);
    st.scores(kop, sa);
    V8 vop[NDB][2];
    vop_at(cur, kGPT - 1, vop);
    st.template next<false>(sbuf(IntC<kGPT - 1>{}), vop, 32, h);
  };
  if (nft > 1) {
    enter_tile(IntC<1>{}, 1);
    {
      V8 kop[KD];
      kop_at(lds1, 0, kop);
      st.scores(kop, sa);
    }
    int t = 1;
    while (true) {  // every tile entered here is followed by a full one
      if (t + 1 >= nft) break;
      tile_body(IntC<1>{}, t++);
      if (t + 1 >= nft) break;
      tile_body(IntC<2>{}, t++);
      if (t + 1 >= nft) break;
      tile_body(IntC<0>{}, t++);
    }
    // last full tile, t = nft - 1
    const unsigned char* cur = buf_rt(t % kNBUF);
    tile_groups(cur);
    V8 vop[NDB][2];
    vop_at(cur, kGPT - 1, vop);
    st.template next<false>(sbuf(IntC<kGPT - 1>{}), vop, 32, h);
  }
  // the partial last tile (1 .. kTJ-1 tokens) after full ones
  const int rem = ntok - nft * kTJ;
  if (nft > 0 && rem > 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const unsigned char* cur = buf_rt(nft % kNBUF);
    for (int grp = 0; grp * 32 < rem; ++grp) {
      const int kvalid = min(32, rem - 32 * grp);
      V8 kop[KD];
      kop_at(cur, grp, kop);
      st.scores(kop, sa);
      V8 vop[NDB][2];
      vop_at(cur, grp, vop);
      if (kvalid == 32) st.template next<false>(sa, vop, 32, h);
      else st.template next<true>(sa, vop, kvalid, h);
    }
  }

  // partials of this chunk: reference m, row sum l and O per latent column
  const int64_t base = ((int64_t)bh * a.nchunks + chunk) * a.Mpad;
  auto write_partials = [&](const auto& t) {
#pragma unroll
    for (int cb = 0; cb < kNC; ++cb) {
      const int col = lat0 + wave * 32 * kNC + cb * 32 + r;
      const float lt = t.row_sum(cb);
      if (h == 0) {
        a.part_m[base + col] = t.reference(cb);
        a.part_l[base + col] = lt;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          const int d0 = 32 * db + 8 * aa + 4 * h;
          if (d0 < D) {
            float* dst = a.part_o + (base + col) * D + d0;
            *reinterpret_cast<f32x4*>(dst) =
                f32x4{t.o[db][cb][4 * aa], t.o[db][cb][4 * aa + 1], t.o[db][cb][4 * aa + 2],
                      t.o[db][cb][4 * aa + 3]};
          }
        }
    }
  };

  // Sums out of range for the fixed reference: recompute this wave's columns
  // exactly, straight from HBM -- first the true column maxima, then the
  // sums, where no probability exceeds 1 and the largest is 1.
  if (!st.overflowed()) {
    write_partials(st);
    return;
  }
  auto kop_g = [&](int G, V8 (&kop)[KD]) {
    const int tok = min(32 * G + r, ntok - 1);
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const int d0 = 16 * kd + 8 * h;
      if (d0 < D) kop[kd] = bitcast_u4<V8>(ldg16(kbase + (n0 + tok) * D + d0));
      else kop[kd] = bitcast_u4<V8>(u32x4{0u, 0u, 0u, 0u});
    }
  };
  auto vop_g = [&](int G, V8 (&vop)[NDB][2]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + r;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        V8 x;
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const int tok = min(32 * G + 16 * kk + 8 * (t8 >> 2) + 4 * h + (t8 & 3), ntok - 1);
          x[t8] = d < D ? vbase[(n0 + tok) * D + d] : (T)0.f;
        }
        vop[db][kk] = x;
      }
    }
  };
  using Exact = FlashTile<T, D, kNC, true>;
  Exact ex;
  ex.reset();
#pragma unroll
  for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) ex.q[cb][kd] = st.q[cb][kd];
  const int ngrp = (ntok + 31) / 32;
  float mx[kNC];
#pragma unroll
  for (int cb = 0; cb < kNC; ++cb) mx[cb] = -__builtin_inff();
  for (int G = 0; G < ngrp; ++G) {
    V8 kop[KD];
    kop_g(G, kop);
    ex.scores(kop, sa);
    Exact::mask(sa, ntok - 32 * G, h);
    float gm[kNC];
    Exact::colmax(sa, gm);
#pragma unroll
    for (int cb = 0; cb < kNC; ++cb) mx[cb] = fmaxf(mx[cb], gm[cb]);
  }
  ex.set_reference(sa, mx);
  for (int G = 0; G < ngrp; ++G) {
    V8 kop[KD];
    kop_g(G, kop);
    ex.scores(kop, sa);
    V8 vop[NDB][2];
    vop_g(G, vop);
    ex.template next<true>(sa, vop, ntok - 32 * G, h);
  }
  write_partials(ex);
}

// fp32 path: one thread per latent row, exact fp32 arithmetic (VALU FMAs),
// tiles of 32 tokens staged in LDS and read as broadcasts.
template <int D>
__global__ __launch_bounds__(512) void encode_split_f32_kernel(EncodeParams a) {
  constexpr int TJ = 32;
  __shared__ float ksm[TJ][D];
  __shared__ float vsm[TJ][D];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int bh = blockIdx.x / a.nchunks;
  const int chunk = blockIdx.x - bh * a.nchunks;
  const int b = bh / a.H, h = bh - b * a.H;
  if (a.gate != nullptr && gate_sigma(a.gate[h]) == 0.f) return;

  const int64_t n0 = (int64_t)chunk * a.chunk_tokens;
  const int64_t n1 = min(a.N, n0 + a.chunk_tokens);
  const float* kb = reinterpret_cast<const float*>(a.k) + (int64_t)bh * a.N * D;
  const float* vb = reinterpret_cast<const float*>(a.v) + (int64_t)bh * a.N * D;
  const float* qb = reinterpret_cast<const float*>(a.q) + b * a.q_b_stride + h * a.q_h_stride;
  const int m = tid;  // latent row (m < Mpad always: blockDim == Mpad)

  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (a.qscale > 0.f) q[d] = m < a.M ? a.qscale * qb[(int64_t)m * D + d] : 0.f;
    else q[d] = qb[(int64_t)m * D + d];
    o[d] = 0.f;
  }
  float mref = -__builtin_inff(), l = 0.f;
  for (int64_t tb = n0; tb < n1; tb += TJ) {
    const int tv = (int)min((int64_t)TJ, n1 - tb);
    for (int e = tid; e < TJ * D; e += nt) {
      const int j = e / D, d = e - j * D;
      ksm[j][d] = j < tv ? kb[(tb + j) * D + d] : 0.f;
      vsm[j][d] = j < tv ? vb[(tb + j) * D + d] : 0.f;
    }
    __syncthreads();
    float s[TJ];
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], ksm[j][d], acc);
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
    for (int j = 0; j < TJ; ++j) {
      const float p = exp2f(s[j] - mref);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, vsm[j][d], o[d]);
    }
    __syncthreads();
  }
  const int64_t base = ((int64_t)bh * a.nchunks + chunk) * a.Mpad + m;
  a.part_m[base] = mref;
  a.part_l[base] = l;
#pragma unroll
  for (int d = 0; d < D; ++d) a.part_o[base * D + d] = o[d];
}

// At D = 64 a workgroup takes at most 8 waves (256 latents): 16 waves would
// be held to 128 VGPRs each and spill ~500 bytes per lane.  Larger M runs
// as several latent blocks along y, each streaming the chunk's tiles.
// The same for the fp16 encode step (separate K and V) at D <= 32, whose
// 16-wave form spills ~160 bytes per lane (it keeps a reference maximum):
// same box, B1 H8 N1048576 M512 D32 fp16, encode 0.90 -> 0.74 ms.  The fp16
// synthesis (K = V, one staged tensor) keeps 16 waves: split, it ran 9%
// slower.
template <int D>
constexpr int kMaxEncWaves = D >= 64 ? 8 : kMaxWaves;

template <typename T, int D>
hipError_t launch_mfma(const EncodeParams& p, hipStream_t s) {
  const bool shared_kv = (p.k == p.v);
  const int all = encode_waves(p.M);
  const int cap = (std::is_same<T, _Float16>::value && !shared_kv) ? 8 : kMaxEncWaves<D>;
  const int nw = all < cap ? all : cap;
  const dim3 grid((unsigned)(p.B * p.H * p.nchunks), (unsigned)(all / nw));
#define FLAREPP_ENC(NWV)                                                                     \
  case NWV:                                                                                  \
    if (shared_kv)                                                                           \
      hipLaunchKernelGGL((encode_split_kernel<T, D, NWV, true>), grid, dim3(64 * NWV), 0, s, p); \
    else                                                                                     \
      hipLaunchKernelGGL((encode_split_kernel<T, D, NWV, false>), grid, dim3(64 * NWV), 0, s, p); \
    break;
  switch (nw) {
    FLAREPP_ENC(1)
    FLAREPP_ENC(2)
    FLAREPP_ENC(4)
    FLAREPP_ENC(8)
#if FLAREPP_ENC_NC == 1
    case 16:
      if constexpr (kMaxEncWaves<D> >= 16) {
        if (shared_kv)
          hipLaunchKernelGGL((encode_split_kernel<T, D, 16, true>), grid, dim3(64 * 16), 0, s, p);
        else if constexpr (!std::is_same<T, _Float16>::value)
          hipLaunchKernelGGL((encode_split_kernel<T, D, 16, false>), grid, dim3(64 * 16), 0, s, p);
      }
      break;
#endif
    default:
      return hipErrorInvalidValue;
  }
#undef FLAREPP_ENC
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const EncodeParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.H * p.nchunks));
  hipLaunchKernelGGL((encode_split_f32_kernel<D>), grid, dim3(p.Mpad), 0, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_mfma_d(int D, const EncodeParams& p, hipStream_t s) {
  switch (D) {
    case 8: return launch_mfma<T, 8>(p, s);
    case 16: return launch_mfma<T, 16>(p, s);
    case 32: return launch_mfma<T, 32>(p, s);
    case 64: return launch_mfma<T, 64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int encode_tile_tokens() { return kTJ; }

int encode_waves(int M) {
  const int w = (M + 32 * kNC - 1) / (32 * kNC);
  return w <= 1 ? 1 : w <= 2 ? 2 : w <= 4 ? 4 : w <= 8 ? 8 : 16;
}

int latent_pad(int M, int dtype) {
  // fp32 path: one thread per latent row in blocks of 64; matrix-core path:
  // 64 latents per wave and a power-of-two wave count.
  if (dtype == kF32) return ((M + 63) / 64) * 64;
  return encode_waves(M) * 32 * kNC;
}

hipError_t launch_encode(int dtype, int D, const EncodeParams& p, hipStream_t s) {
  if (dtype == kBF16) return launch_mfma_d<__bf16>(D, p, s);
  if (dtype == kF16) return launch_mfma_d<_Float16>(D, p, s);
  switch (D) {
    case 8: return launch_f32<8>(p, s);
    case 16: return launch_f32<16>(p, s);
    case 32: return launch_f32<32>(p, s);
    case 64: return launch_f32<64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace flarepp
