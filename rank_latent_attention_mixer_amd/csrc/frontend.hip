// Front end of the FLARE++ block on the gfx950 matrix cores: the three
// input projections k0, k, v of the token features and the head-wise
// normalisation of k0 (issue #2024, "Changes from v1 to v2": three
// projections, the synthesis keys and values shared; the synthesis call
// normalised head by head), and the same normalisation of the seeds q0.
//
// One launch computes all three projections as one GEMM over the
// concatenated output features F = 3 H D:  out[t][j] = x[t] . W_p[r] + b_p[r]
// with p = j / (H D), r = j % (H D), W_p in the [H D, C] layout of a linear
// layer.  The epilogue adds the bias, applies u / sqrt(mean(u^2) + eps) * g
// to every D-feature head group of k0, and writes each group straight into
// its [B, H, N, D] tensor, so the projections are never stored token-major.
//
// Tiling: a workgroup (4 waves) owns 128 tokens x 128 features; each wave a
// 64 x 64 sub-tile as 2 x 2 products of 32 x 32 on v_mfma_f32_32x32x16,
// evaluated transposed (features as rows, tokens as columns) so each lane
// holds 16 features of one token -- the head's sum of squares is a lane sum
// plus one cross-half shuffle.  K runs over C in steps of 32; the W and x
// tiles of each step go HBM -> LDS by direct loads (no registers) into three
// rotating buffers, two steps ahead of the matrix cores.  The output tile is
// staged through LDS so that each store instruction writes 1 KB contiguous
// of a head's [N, D] block.  Workgroups are renumbered so the feature tiles
// of one token tile run on one XCD and share its L2 copy of x.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "flarepp_device.hpp"
#include "frontend.hpp"
#include "kernels.hpp"

namespace flarepp {

namespace {

constexpr int kFeTile = 128;   // tokens and features per workgroup
constexpr int kFeK = 32;       // K (input features) per LDS step
constexpr int kFeRowB = kFeK * 2;            // bytes per tile row (4 chunks of 16)
constexpr int kFeTileB = kFeTile * kFeRowB;  // bytes per operand tile (8 KB)
constexpr int kFeStageB = 2 * kFeTileB;      // W and x tiles of one K step
constexpr int kFeBufs = 3;                   // K steps: 2 loading while 1 is in use
constexpr int kXcds = 8;

// Byte offset of 16-byte chunk c of tile row `row`: the chunk index is XOR-ed
// with (row / 4) % 4, so the 16 lanes of a quarter-wave reading rows
// r..r+15 at one logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ int fe_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int fe_off(int row, int c) { return row * kFeRowB + ((c ^ fe_swz(row)) << 4); }

// s_waitcnt with vmcnt <= n (expcnt and lgkmcnt left at their maxima)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | n);
}

// Three workgroups per CU (48 KB of LDS each, registers capped to match):
// the K loop is bound by load latency, so occupancy is what hides it.
template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void frontend_kernel(FrontendParams a) {
  typedef typename Pack8<T>::type V8;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kFeBufs * kFeStageB];  // 48 KB
  static_assert(kFeBufs * kFeStageB >= 4 * 64 * 128, "output staging reuses the K buffers");

  const int64_t F = 3 * (int64_t)a.H * D;
  const int ftiles = (int)((F + kFeTile - 1) / kFeTile);
  // XCD-aware renumbering: workgroup g runs on XCD g % 8; give each XCD a
  // contiguous range of (token tile, feature tile) pairs, feature fastest,
  // so the feature tiles of a token tile share one L2 copy of its x rows
  const int64_t G = (int64_t)gridDim.x;
  const int64_t per_xcd = G / kXcds;                      // G is a multiple of 8
  const int64_t g = blockIdx.x;
  const int64_t pair = (g % kXcds) * per_xcd + g / kXcds;
  const int64_t ttile = pair / ftiles;
  const int ftile = (int)(pair - ttile * ftiles);
  const int64_t t0 = ttile * kFeTile;
  if (t0 >= a.T) return;  // padding workgroups (uniform)
  const int f0 = ftile * kFeTile;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int fo = 64 * (wave & 1), to = 64 * (wave >> 1);  // the wave's sub-tile
  const int HDi = a.H * D, Fi = 3 * HDi;  // < 2^31 (checked at the boundary)

  // HBM -> LDS with no registers: a wave load moves 1 KB, lane i's 16 bytes
  // landing at byte 16 i of it.  Each wave issues 4 of the 16 loads of a K
  // step (W tile then x tile); the lane's row and chunk are the inverse of
  // the swizzle.  Rows past the matrix repeat its last row (their outputs
  // are not stored); K past C reads a valid column and is zeroed at use.
  const T* src_row[4];
  int dst_off[4], lchunk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ld = wave * 4 + i;               // 0..15: 8 for W, 8 for x
    const int ten = ld >> 3, li = ld & 7;
    const int o = li * 1024 + 16 * lane;       // byte within the operand tile
    const int row = o / kFeRowB;
    lchunk[i] = ((o % kFeRowB) >> 4) ^ fe_swz(row);
    dst_off[i] = ten * kFeTileB + li * 1024;
    if (ten == 0) {
      const int j = min(f0 + row, Fi - 1);
      const int p = j / HDi;
      src_row[i] = reinterpret_cast<const T*>(a.w[p]) + (int64_t)(j - p * HDi) * a.C;
    } else {
      const int64_t t = min(t0 + row, a.T - 1);
      src_row[i] = reinterpret_cast<const T*>(a.x) + t * a.C;
    }
  }
  const int nk = (int)((a.C + kFeK - 1) / kFeK);
  auto issue = [&](int ks) {
    unsigned char* stage = lds + (ks % kFeBufs) * kFeStageB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t k = (int64_t)ks * kFeK + 8 * lchunk[i];
      if (k >= a.C) k = 0;  // zeroed at use
      global_to_lds16(src_row[i] + k, stage + dst_off[i]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int fs = 0; fs < 2; ++fs)
#pragma unroll
    for (int ts = 0; ts < 2; ++ts)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fs][ts][v] = 0.f;

  issue(0);
  if (nk > 1) issue(1);
  for (int ks = 0; ks < nk; ++ks) {
    // step ks's loads are done once at most those of step ks+1 remain
    if (ks + 1 < nk) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    // ... in every wave; the barrier also retires all reads of step ks-1,
    // whose buffer now receives step ks+2
    __syncthreads();
    if (ks + 2 < nk) issue(ks + 2);
    const unsigned char* bw = lds + (ks % kFeBufs) * kFeStageB;
    const unsigned char* bx = bw + kFeTileB;
#pragma unroll
    for (int kk = 0; kk < kFeK / 16; ++kk) {
      const int c = 2 * kk + h;  // this lane's 16-byte chunk of the K step
      const bool kin = (int64_t)ks * kFeK + 8 * c < a.C;
      V8 wa[2], xb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int fr = fo + 32 * s + r, tr = to + 32 * s + r;
        wa[s] = *reinterpret_cast<const V8*>(bw + fe_off(fr, c));
        if (!kin) wa[s] = bitcast_u4<V8>(u32x4{0u, 0u, 0u, 0u});
        xb[s] = *reinterpret_cast<const V8*>(bx + fe_off(tr, c));
      }
#pragma unroll
      for (int fs = 0; fs < 2; ++fs)
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) acc[fs][ts] = mfma_32x32x16(wa[fs], xb[ts], acc[fs][ts]);
    }
  }

  // Epilogue.  The lane holds features fo + 32 fs + 8 aa + 4 h + i of token
  // to + 32 ts + r.  Bias, then the head-wise normalisation of k0, then the
  // values go through LDS (the wave's 64 x 64 block, [token][feature], 16-byte
  // chunks XOR-swizzled by row) so that every store writes 1 KB contiguous.
  constexpr int NHD = 64 / D;  // heads in the wave's 64 features
  float bias[2][16], gain[2][16];
  bool norm_grp[2][4];
#pragma unroll
  for (int fs = 0; fs < 2; ++fs)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const int j = f0 + fo + 32 * fs + 8 * aa + 4 * h;
      int p = -1, rr = 0;
      if (j < Fi) {
        p = j / HDi;
        rr = j - p * HDi;
      }
      norm_grp[fs][aa] = p == 0 && a.normalize;
      const T* bp = p >= 0 ? reinterpret_cast<const T*>(a.b[p]) : nullptr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bias[fs][4 * aa + i] = bp ? (float)bp[rr + i] : 0.f;
        gain[fs][4 * aa + i] = (norm_grp[fs][aa] && a.g)
                                   ? (float)reinterpret_cast<const T*>(a.g)[rr + i] : 1.f;
      }
    }
  __syncthreads();  // every wave is done reading the K-step buffers
  unsigned char* stg = lds + wave * (64 * 128);
  auto stg_off = [](int row, int byte) { return row * 128 + ((((byte >> 4) ^ (row & 7)) << 4) | (byte & 15)); };
#pragma unroll
  for (int ts = 0; ts < 2; ++ts) {
    float ss[NHD];
#pragma unroll
    for (int q = 0; q < NHD; ++q) ss[q] = 0.f;
#pragma unroll
    for (int fs = 0; fs < 2; ++fs)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float val = acc[fs][ts][v] + bias[fs][v];
        acc[fs][ts][v] = val;
        ss[(32 * fs + 8 * (v >> 2)) / D] = fmaf(val, val, ss[(32 * fs + 8 * (v >> 2)) / D]);
      }
#pragma unroll
    for (int q = 0; q < NHD; ++q) ss[q] += __shfl_xor(ss[q], 32);
    const int row = 32 * ts + r;
#pragma unroll
    for (int fs = 0; fs < 2; ++fs)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const float inv = norm_grp[fs][aa]
                              ? rsqrtf(ss[(32 * fs + 8 * aa) / D] * (1.f / D) + a.eps) : 1.f;
        typename Pack8<T>::pair lo, hi;
        lo[0] = (T)(acc[fs][ts][4 * aa] * inv * gain[fs][4 * aa]);
        lo[1] = (T)(acc[fs][ts][4 * aa + 1] * inv * gain[fs][4 * aa + 1]);
        hi[0] = (T)(acc[fs][ts][4 * aa + 2] * inv * gain[fs][4 * aa + 2]);
        hi[1] = (T)(acc[fs][ts][4 * aa + 3] * inv * gain[fs][4 * aa + 3]);
        const int byte = 2 * (32 * fs + 8 * aa + 4 * h);
        *reinterpret_cast<u32x2*>(stg + stg_off(row, byte)) =
            u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
      }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  // Stores: per head of the wave, its D features of the wave's 64 tokens;
  // lane -> (token, 16-byte chunk), consecutive lanes consecutive bytes.
  constexpr int CPH = D / 8;         // 16-byte chunks per token row of a head
  constexpr int TPI = 64 / CPH;      // tokens per store instruction
  const int64_t tw = t0 + to;        // first token of the wave
#pragma unroll
  for (int hh = 0; hh < NHD; ++hh) {
    const int j = f0 + fo + hh * D;  // first feature of the head
    if (j >= Fi) break;
    const int p = j / HDi;
    const int hd = (j - p * HDi) / D;
    T* outp = reinterpret_cast<T*>(a.out[p]);
#pragma unroll
    for (int q = 0; q < CPH; ++q) {
      const int u = q * TPI + lane / CPH, c = lane % CPH;
      const int64_t t = tw + u;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stg + stg_off(u, 2 * hh * D + 16 * c));
      if (t < a.T) {
        const int64_t bb = t / a.N, n = t - bb * a.N;
        *reinterpret_cast<u32x4*>(outp + ((bb * a.H + hd) * a.N + n) * D + 8 * c) = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Narrow inputs (C <= 256, a multiple of 64): weights resident in registers.
// ---------------------------------------------------------------------------
// A workgroup owns 256 consecutive output features; each of its 4 waves
// holds the weights of its 64 features for all C inputs in registers (the
// A operands of 2 feature tiles x C/16 steps: C/2 VGPRs), loaded once.
// The workgroup then streams a range of tokens in blocks of 32: each x
// block goes HBM -> LDS by direct loads (three buffers, two blocks ahead)
// and every wave multiplies it by its resident weights, so a block is read
// from L2 once per 256 features and the weights are never re-read.  The
// epilogue of block b (bias, k0 normalisation, conversion) is staged in LDS
// and stored during block b+1.  The two kinds of memory traffic are kept
// in separate waves, because gfx9 counts loads and stores on one counter and
// a wait for loads would also wait for every older store: the even waves
// issue the direct loads (and wait for them) and store nothing, the odd
// waves store their own and their even neighbour's results and load
// nothing.  The workgroups of the feature groups of one token range are
// numbered onto one XCD so they share its L2 copy of x.
constexpr int kWrFeat = 256;         // features per workgroup
// Workgroup numbering: nnorm feature groups (the first ones, which hold
// normalised features) and rx token ranges per XCD for every group.
struct WresSplit {
  int nnorm, rx;
};
constexpr int kWrTok = 32;           // tokens per block
constexpr int kWrBufs = 3;
constexpr int kWrStageB = 32 * 128;  // 32 tokens x 64 features x 2 B

// Byte offset of logical 16-byte chunk c of row `row` of an x block (rows of
// 2C bytes).  The 16 lanes of a quarter-wave read rows r..r+15 (r a multiple
// of 16) at one logical chunk; the XOR spreads them over the 16 slots of 16
// bytes in 256: rows of 512 or 256 bytes use row % 16, rows of 384 or 128
// bytes (two rows per 256-byte period) use (row / 2) % 8.
template <int C>
__device__ __forceinline__ int wr_swz(int row) { return (C % 128 == 0) ? (row & 15) : ((row >> 1) & 7); }
template <int C>
__device__ __forceinline__ int wr_off(int row, int c) { return row * (2 * C) + ((c ^ wr_swz<C>(row)) << 4); }
// Direct load `slot` of an x block fills LDS bytes [1 KB slot, +1 KB), lane
// i's 16 bytes at 16 i: the token row and element column it must read (the
// inverse of the swizzle).
template <int C>
__device__ __forceinline__ void wr_load_slot(int slot, int lane, int& row, int& col) {
  const int o = slot * 1024 + 16 * lane;
  row = o / (2 * C);
  col = 8 * (((o - row * 2 * C) >> 4) ^ wr_swz<C>(row));
}
// staging: [token][feature] rows of 128 bytes, 16-byte chunks XOR-ed by row
__device__ __forceinline__ int stg_off(int row, int byte) {
  return row * 128 + ((((byte >> 4) ^ (row & 7)) << 4) | (byte & 15));
}

// s_waitcnt vmcnt(n) for n < 64 (expcnt and lgkmcnt left at their maxima)
template <int n>
__device__ __forceinline__ void wait_vmcnt64() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// Per-wave state of the narrow-input kernel.
template <typename T, int D, int C>
struct WresWave {
  typedef typename Pack8<T>::type V8;
  static constexpr int KS = C / 16;
  static constexpr int QE = kWrTok * 2 * C / 1024 / 2;  // direct loads per even wave per block
  V8 w[2][KS];                 // resident weights (A operands)
  int lane, wave, h, r, f0, fo, HDi, Fi;
  bool any_norm;               // some group of the wave is normalised (uniform)
};

// Stores of the staged block of the wave owning features fo_src: per head,
// its D features of the block's 32 tokens, lane -> (token, 16-byte chunk),
// consecutive lanes consecutive bytes (1 KB per store instruction).
template <typename T, int D, int C>
__device__ __forceinline__ void wres_store(const FrontendParams& a, const WresWave<T, D, C>& s,
                                           const unsigned char* __restrict__ stg, int fo_src,
                                           int64_t tb, int64_t bb0, int64_t n0) {
  constexpr int NHD = 64 / D;
  constexpr int CPH = D / 8;     // 16-byte chunks per token row of a head
  constexpr int TPI = 64 / CPH;  // tokens per store instruction
  const bool inside = n0 + kWrTok <= a.N && tb + kWrTok <= a.T;  // one batch, all valid
#pragma unroll
  for (int hh = 0; hh < NHD; ++hh) {
    const int j = s.f0 + fo_src + hh * D;  // wave-uniform
    if (j >= s.Fi) break;
    const int p = j / s.HDi;
    const int hd = (j - p * s.HDi) / D;
    T* outp = reinterpret_cast<T*>(p == 0 ? a.out[0] : p == 1 ? a.out[1] : a.out[2]);
    T* base = outp + ((bb0 * a.H + hd) * a.N + n0) * D;
#pragma unroll
    for (int q = 0; q < kWrTok / TPI; ++q) {
      const int u = q * TPI + s.lane / CPH, c = s.lane % CPH;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stg + stg_off(u, 2 * hh * D + 16 * c));
      // non-temporal: the outputs are not read again here, and streaming
      // them past the L2 leaves it to the x rows the other feature groups
      // of the token range still read
      if (inside) {  // uniform base, per-lane 32-bit offset
        __builtin_nontemporal_store(
            val, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + (unsigned)(2 * (u * D + 8 * c))));
      } else if (tb + u < a.T) {
        int64_t bb = bb0, n = n0 + u;
        while (n >= a.N) { n -= a.N; ++bb; }
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(outp + ((bb * a.H + hd) * a.N + n) * D + 8 * c));
      }
    }
  }
}

// Direct load i (0..QE-1) of an even wave for the block starting at token tb.
template <typename T, int D, int C>
__device__ __forceinline__ void wres_dma_one(const FrontendParams& a, const WresWave<T, D, C>& s,
                                             unsigned char* __restrict__ dst, int64_t tb, int i) {
  constexpr int QE = WresWave<T, D, C>::QE;
  int row, col;
  wr_load_slot<C>(QE * (s.wave >> 1) + i, s.lane, row, col);
  const int64_t t = min(tb + row, a.T - 1);  // rows past T: not stored
  global_to_lds16(reinterpret_cast<const T*>(a.x) + t * C + col, dst + (QE * (s.wave >> 1) + i) * 1024);
}

// One block step after its barrier: the odd waves store the staged block
// blk-1 (theirs, from `stg`, and their even neighbour's, from `stg_nbr`)
// and the even waves start the direct loads of block blk+2 into `next` (if
// any); then every active wave multiplies block blk in `cur` by its weights
// and stages the result in `stg` (odd waves: after reading block blk-1
// from it).  The
// pointers are restrict-qualified so that the compiler's wait insertion can
// tell the LDS reads from the direct loads into `next` (else it waits for
// those loads before the first LDS read, undoing the prefetch); the caller
// waits for block blk's own loads.
template <typename T, int D, int C>
__device__ __forceinline__ void wres_step(const FrontendParams& a, const WresWave<T, D, C>& s,
                                          const unsigned char* __restrict__ cur,
                                          unsigned char* __restrict__ next,
                                          unsigned char* __restrict__ stg,
                                          const unsigned char* __restrict__ stg_nbr,
                                          const float* __restrict__ tab, bool store_prev,
                                          int64_t ptb, int64_t pbb, int64_t pn, int64_t next_tb,
                                          bool active, bool nbr_active) {
  typedef typename Pack8<T>::type V8;
  constexpr int KS = C / 16, QE = WresWave<T, D, C>::QE, NHD = 64 / D;
  const bool odd = s.wave & 1;
  if (odd && store_prev) {
    if (nbr_active) wres_store<T, D, C>(a, s, stg_nbr, s.fo - 64, ptb, pbb, pn);
    if (active) wres_store<T, D, C>(a, s, stg, s.fo, ptb, pbb, pn);
  }
  if (!odd && next)
#pragma unroll
    for (int i = 0; i < QE; ++i) wres_dma_one<T, D, C>(a, s, next, next_tb, i);
  if (!active) return;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): no scalar loads left in flight
  // the bias is the products' initial value: lane feature fo + 32 fs + 8 aa + 4 h + i
  f32x16 acc[2];
#pragma unroll
  for (int fs = 0; fs < 2; ++fs)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(tab + s.fo + 32 * fs + 8 * aa + 4 * s.h);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[fs][4 * aa + i] = bv[i];
    }
  // x operands read two steps ahead of their products, no further (the
  // resident weights leave few registers).  The swizzle permutes chunks
  // only within periods of 2P, so P addresses and immediate offsets serve
  // all C/16 steps.
  const unsigned char* rowp = cur + s.r * (2 * C);
  auto rd = [&](int k) {
    constexpr int P = (C % 128 == 0) ? 8 : 4;  // steps per swizzle period (2P chunks)
    return *reinterpret_cast<const V8*>(rowp + (k / P) * 32 * P +
                                        (((2 * (k % P) + s.h) ^ wr_swz<C>(s.r)) << 4));
  };
  // (one step ahead only at D = 64, C = 256, whose epilogue needs the room)
  constexpr int LA = (D == 64 && C == 256) ? 1 : 2;
  V8 x0 = rd(0), x1 = LA > 1 ? rd(1) : x0;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const V8 x2 = k + LA < KS ? rd(k + LA) : x1;
    acc[0] = mfma_32x32x16(s.w[0][k], x0, acc[0]);
    acc[1] = mfma_32x32x16(s.w[1][k], x0, acc[1]);
    __builtin_amdgcn_sched_barrier(0);
    if (LA > 1) {
      x0 = x1;
      x1 = x2;
    } else {
      x0 = x2;
    }
  }
  // epilogue: the lane holds features fo + 32 fs + 8 aa + 4 h + i of token r
  if (s.any_norm) {
    float ss[NHD];
#pragma unroll
    for (int q = 0; q < NHD; ++q) ss[q] = 0.f;
#pragma unroll
    for (int fs = 0; fs < 2; ++fs)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        ss[(32 * fs + 8 * (v >> 2)) / D] = fmaf(acc[fs][v], acc[fs][v], ss[(32 * fs + 8 * (v >> 2)) / D]);
#pragma unroll
    for (int q = 0; q < NHD; ++q) ss[q] += __shfl_xor(ss[q], 32);
#pragma unroll
    for (int fs = 0; fs < 2; ++fs)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(tab + kWrFeat + s.fo + 32 * fs + 8 * aa + 4 * s.h);
        // normalised: the group's features belong to k0 (the wave's are all
        // projected features once any_norm holds)
        const bool ng = s.f0 + s.fo + 32 * fs + 8 * aa + 4 * s.h < s.HDi;
        const float inv = ng ? rsqrtf(ss[(32 * fs + 8 * aa) / D] * (1.f / D) + a.eps) : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[fs][4 * aa + i] *= inv * gv[i];
        __builtin_amdgcn_sched_barrier(0);  // one gain vector live at a time
      }
  }
#pragma unroll
  for (int fs = 0; fs < 2; ++fs)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      typename Pack8<T>::pair lo, hi;
      lo[0] = (T)acc[fs][4 * aa];
      lo[1] = (T)acc[fs][4 * aa + 1];
      hi[0] = (T)acc[fs][4 * aa + 2];
      hi[1] = (T)acc[fs][4 * aa + 3];
      *reinterpret_cast<u32x2*>(stg + stg_off(s.r, 2 * (32 * fs + 8 * aa + 4 * s.h))) =
          u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    }
}

template <typename T, int D, int C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void frontend_wres_kernel(FrontendParams a, WresSplit sp) {
  typedef typename Pack8<T>::type V8;
  using S = WresWave<T, D, C>;
  constexpr int KS = S::KS, QE = S::QE;
  constexpr int BLKB = kWrTok * 2 * C;     // bytes of one x block
  static_assert(C % 64 == 0 && C <= 256 && QE >= 1, "narrow-input path");
  // LDS: x blocks [kWrBufs][BLKB]; staging: even waves two blocks (their
  // neighbour stores block b-1 while they stage block b), odd waves one;
  // bias and gain table
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* xbuf = lds;
  unsigned char* stg_all = lds + kWrBufs * BLKB;                   // [2 pairs][3 blocks]
  float* tab = reinterpret_cast<float*>(stg_all + 6 * kWrStageB);  // bias[256], gain[256]

  S s;
  s.HDi = a.H * D;
  s.Fi = 3 * s.HDi;
  const int FG = (s.Fi + kWrFeat - 1) / kWrFeat;
  const int g = blockIdx.x;
  const int xcd = g % kXcds, slot = g / kXcds;
  // the feature groups that normalise (the first sp.nnorm) cost ~1.3x a
  // plain group per block and take the first slots of every XCD, the plain
  // groups the rest; the plain groups of one token range sit side by side
  const int nplain = FG - sp.nnorm;
  const bool norm_slot = slot < sp.nnorm * sp.rx;
  const int t = norm_slot ? slot : slot - sp.nnorm * sp.rx;
  const int ncls = norm_slot ? sp.nnorm : nplain;
  const int fg = norm_slot ? t % ncls : sp.nnorm + t % ncls;
  const int range = (t / ncls) * kXcds + xcd;
  const int64_t nblk = (a.T + kWrTok - 1) / kWrTok;
  const int64_t R = (int64_t)kXcds * sp.rx;
  const int64_t per = (nblk + R - 1) / R;
  const int64_t b0 = range * per;
  const int64_t nb = min(b0 + per, nblk) - b0;
  if (nb <= 0) return;  // uniform: more ranges than blocks

  const int tid = threadIdx.x;
  s.lane = tid & 63;
  s.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  s.h = s.lane >> 5;
  s.r = s.lane & 31;
  s.f0 = fg * kWrFeat;
  s.fo = 64 * s.wave;
  const bool active = s.f0 + s.fo < s.Fi;                          // wave-uniform
  const bool nbr_active = (s.wave & 1) && s.f0 + s.fo - 64 < s.Fi;  // odd waves' neighbour
  s.any_norm = a.normalize && s.f0 + s.fo < s.HDi;

  // bias and gain of the workgroup's features (gain 1 outside normalised k0)
  for (int i = tid; i < kWrFeat; i += 256) {
    const int j = s.f0 + i;
    float bv = 0.f, gv = 1.f;
    if (j < s.Fi) {
      const int p = j / s.HDi, rr = j - p * s.HDi;
      const void* bp = p == 0 ? a.b[0] : p == 1 ? a.b[1] : a.b[2];
      if (bp) bv = (float)reinterpret_cast<const T*>(bp)[rr];
      if (p == 0 && a.normalize && a.g) gv = (float)reinterpret_cast<const T*>(a.g)[rr];
    }
    tab[i] = bv;
    tab[kWrFeat + i] = gv;
  }

  // resident weights: lane row = feature f0 + fo + 32 fs + r, chunk 2 k + h
#pragma unroll
  for (int fs = 0; fs < 2; ++fs) {
    const int j = min(s.f0 + s.fo + 32 * fs + s.r, s.Fi - 1);
    const int p = j / s.HDi;
    const T* wr = reinterpret_cast<const T*>(p == 0 ? a.w[0] : p == 1 ? a.w[1] : a.w[2]) +
                  (int64_t)(j - p * s.HDi) * C;
#pragma unroll
    for (int k = 0; k < KS; ++k) s.w[fs][k] = *reinterpret_cast<const V8*>(wr + 16 * k + 8 * s.h);
  }
  // the weights are in before the loop (else the wait for them, placed in
  // the loop, would also wait for every direct load in flight)
  wait_vmcnt64<0>();
  __syncthreads();  // the table is written

  const bool even = !(s.wave & 1);
  if (even) {
#pragma unroll
    for (int i = 0; i < QE; ++i) wres_dma_one<T, D, C>(a, s, xbuf, b0 * kWrTok, i);
    if (nb > 1)
#pragma unroll
      for (int i = 0; i < QE; ++i) wres_dma_one<T, D, C>(a, s, xbuf + BLKB, (b0 + 1) * kWrTok, i);
  }
  // staging of the wave pair: the even wave's two blocks, then the odd wave's
  unsigned char* stg_even = stg_all + (s.wave >> 1) * 3 * kWrStageB;
  unsigned char* stg_odd = stg_even + 2 * kWrStageB;
  int64_t tb = b0 * kWrTok;
  int64_t bb0 = tb / a.N, n0 = tb - bb0 * a.N;
  int64_t ptb = 0, pbb = 0, pn = 0;  // the staged block
  for (int64_t blk = 0; blk < nb; ++blk) {
    // Even waves: block blk's loads are done once at most the QE loads of
    // block blk+1 (the last ones issued; no stores in between) remain.  The
    // barrier then says every part of block blk is in and every wave is done
    // with block blk-1, whose buffer receives block blk+2.  (No
    // __syncthreads: its fence would wait for the loads in flight.)
    if (even) {
      if (blk + 1 < nb) wait_vmcnt64<QE>();
      else wait_vmcnt64<0>();
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int cb = (int)(blk % kWrBufs);
    unsigned char* next = blk + 2 < nb ? xbuf + ((cb + 2) % kWrBufs) * BLKB : nullptr;
    const int par = (int)(blk & 1);
    wres_step<T, D, C>(a, s, xbuf + cb * BLKB, next, even ? stg_even + par * kWrStageB : stg_odd,
                       stg_even + (par ^ 1) * kWrStageB, tab, blk > 0, ptb, pbb, pn,
                       (b0 + blk + 2) * kWrTok, active, nbr_active);
    asm volatile("" ::: "memory");
    ptb = tb; pbb = bb0; pn = n0;
    tb += kWrTok;
    n0 += kWrTok;
    while (n0 >= a.N) { n0 -= a.N; ++bb0; }
  }
  // the last block: its staging is written by every wave
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (!even) {
    if (nbr_active) wres_store<T, D, C>(a, s, stg_even + (int)((nb - 1) & 1) * kWrStageB, s.fo - 64, ptb, pbb, pn);
    if (active) wres_store<T, D, C>(a, s, stg_odd, s.fo, ptb, pbb, pn);
  }
}

size_t wres_lds_bytes(int C) {
  return (size_t)kWrBufs * kWrTok * 2 * C + 6 * kWrStageB + 2 * kWrFeat * sizeof(float);
}

template <typename T, int D, int C>
hipError_t wres_launch(const FrontendParams& p, hipStream_t s) {
  const int F = 3 * p.H * D;
  const int FG = (F + kWrFeat - 1) / kWrFeat;
  // about two resident workgroups per CU (256 CUs).  The normalising groups
  // (sum of squares, reciprocal root and two multiplies per value) are the
  // slowest; numbered first, they measured 0.719 -> 0.693 ms at the
  // million-token width, against 0.70-0.71 ms for giving them more, shorter
  // ranges in proportion to their cost.
  WresSplit sp;
  sp.nnorm = p.normalize ? std::min(FG, (p.H * D + kWrFeat - 1) / kWrFeat) : 0;
  sp.rx = std::max(1, 512 / (kXcds * FG));
  const int64_t G = (int64_t)kXcds * FG * sp.rx;
  if (G > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = wres_lds_bytes(C);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)frontend_wres_kernel<T, D, C>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((frontend_wres_kernel<T, D, C>), dim3((unsigned)G), dim3(256), lds, s, p, sp);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t wres_c(const FrontendParams& p, hipStream_t s) {
  switch (p.C) {
    case 64: return wres_launch<T, D, 64>(p, s);
    case 128: return wres_launch<T, D, 128>(p, s);
    case 192: return wres_launch<T, D, 192>(p, s);
    case 256: return wres_launch<T, D, 256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Seeds: one wave per (h, m) row, u / sqrt(mean(u^2) + eps) * g.
template <typename T>
__global__ __launch_bounds__(256) void seed_norm_kernel(SeedNormParams a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int d = threadIdx.x & 63;
  if (row >= (int64_t)a.H * a.M) return;
  const int hd = (int)(row / a.M);
  const bool live = d < a.D;
  const float u = live ? (float)reinterpret_cast<const T*>(a.q0)[row * a.D + d] : 0.f;
  float ss = u * u;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (!live) return;
  const float g = a.g ? (float)reinterpret_cast<const T*>(a.g)[hd * a.D + d] : 1.f;
  reinterpret_cast<T*>(a.out)[row * a.D + d] = (T)(u * rsqrtf(ss / a.D + a.eps) * g);
}

template <typename T>
hipError_t frontend_d(int D, const FrontendParams& p, hipStream_t s) {
  if (p.C % 64 == 0 && p.C <= 256) {
    switch (D) {
      case 16: return wres_c<T, 16>(p, s);
      case 32: return wres_c<T, 32>(p, s);
      case 64: return wres_c<T, 64>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int64_t F = 3 * (int64_t)p.H * D;
  const int64_t tiles = ((p.T + kFeTile - 1) / kFeTile) * ((F + kFeTile - 1) / kFeTile);
  const int64_t G = (tiles + kXcds - 1) / kXcds * kXcds;
  if (G > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)G), block(256);
  switch (D) {
    case 16: hipLaunchKernelGGL((frontend_kernel<T, 16>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((frontend_kernel<T, 32>), grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((frontend_kernel<T, 64>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_frontend(int dtype, int D, const FrontendParams& p, hipStream_t s) {
  return dtype == kBF16 ? frontend_d<__bf16>(D, p, s) : frontend_d<_Float16>(D, p, s);
}

hipError_t launch_seed_norm(int dtype, const SeedNormParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.H * p.M;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (dtype == kBF16) hipLaunchKernelGGL(seed_norm_kernel<__bf16>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(seed_norm_kernel<_Float16>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace flarepp
