// Front end of the FLARE++ block on the gfx950 matrix cores: the three
// input projections k0, k, v of the token features and the head-wise
// normalisation of k0 (FLARE.py README, "FLARE++": three projections, the
// synthesis keys and values shared; the synthesis call normalised head by
// head), and the same normalisation of the seeds q0.
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
