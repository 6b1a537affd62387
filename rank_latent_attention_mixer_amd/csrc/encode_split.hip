// Split-N encoder: per token chunk, the online-softmax partials of
//   z = softmax_rows(scale q k^T) v        (encode, FLARE.py README "FLARE++")
//   q_dyn = softmax_rows(scale q0 k0^T) k0 (synthesis, keys = values = k0)
// as (reference m, row sum l, unnormalised output O) per latent row, which
// the combine kernel merges with log-sum-exp weights (issue #2024,
// "Multi-GPU context parallelism": exact token-sharded encoder).
//
// One workgroup = one (batch, head, token chunk).  Its waves split the
// latents (64 per wave); every wave consumes the same K/V tiles, staged in
// LDS once per workgroup: K in natural [token][d] layout, V transposed to
// [d][key slot] while it is written (the P.V product contracts over tokens,
// so the matrix-core operand needs V with tokens along k).  Tiles of 64
// tokens are double-buffered: the global loads of tile t+1 are in flight
// while tile t is computed.
#include "flash_tile.hpp"
#include "kernels.hpp"

namespace flarepp {

namespace {

constexpr int kNC = 4;        // 16-column blocks per wave -> 64 latents per wave
constexpr int kTJ = 64;       // tokens per LDS tile

template <typename T, int D, int NW, bool SHARED_KV>
__global__ __launch_bounds__(64 * NW) void encode_split_kernel(EncodeParams a) {
  using Tile = FlashTile<T, D, kNC>;
  using V8 = typename Tile::V8;
  constexpr int KD = Tile::KD, DV = Tile::DV, NDB = Tile::NDB;
  constexpr int KP = (D < 8 ? 8 : D) + 8;   // K row pitch (elements), 16-byte multiple
  constexpr int VP = kTJ + 8;               // V^T row pitch
  constexpr int NT = 64 * NW;
  constexpr int G8 = D / 8;                 // 16-byte groups per token row
  constexpr int U = (kTJ / 2) * G8;         // load units per tile: 2 rows x 16 bytes
  constexpr int UPT = (U + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) T ks[2][kTJ * KP];
  __shared__ __attribute__((aligned(16))) T vt[2][DV * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int bh = blockIdx.x / a.nchunks;
  const int chunk = blockIdx.x - bh * a.nchunks;
  const int b = bh / a.H, h = bh - b * a.H;

  if (a.gate != nullptr && gate_sigma(a.gate[h]) == 0.f) return;  // closed gate: no synthesis

  const int64_t n0 = (int64_t)chunk * a.chunk_tokens;
  const int64_t n1 = min(a.N, n0 + a.chunk_tokens);
  const int ntiles = (int)((n1 - n0 + kTJ - 1) / kTJ);
  const T* kbase = reinterpret_cast<const T*>(a.k) + (int64_t)bh * a.N * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (int64_t)bh * a.N * D;

  if constexpr (D < 16) {
    // value rows D..15 of both buffers stay zero for the whole kernel
    for (int e = tid; e < 2 * (DV - D) * VP; e += NT) {
      const int buf = e / ((DV - D) * VP), rem = e - buf * (DV - D) * VP;
      vt[buf][D * VP + rem] = (T)0.f;
    }
  }

  Tile st;
  st.reset();
  {
    const T* qb = reinterpret_cast<const T*>(a.q) + b * a.q_b_stride + h * a.q_h_stride;
#pragma unroll
    for (int cb = 0; cb < kNC; ++cb) {
      const int col = wave * 16 * kNC + cb * 16 + r;
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) {
        const int d0 = 32 * kd + 8 * g;
        if (d0 < D) st.q[cb][kd] = bitcast_u4<V8>(ldg16(qb + (int64_t)col * D + d0));
        else st.q[cb][kd] = bitcast_u4<V8>(u32x4{0u, 0u, 0u, 0u});
      }
    }
  }

  u32x4 pk[UPT][2], pv[UPT][2];
  auto load_tile = [&](int t) {
    const int64_t tb = n0 + (int64_t)t * kTJ;
#pragma unroll
    for (int uu = 0; uu < UPT; ++uu) {
      const int u = tid + uu * NT;
      if (U % NT == 0 || u < U) {
        const int pr = u / G8, e = u - pr * G8;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int64_t n = tb + 2 * pr + rr;
          if (n < n1) {
            pk[uu][rr] = ldg16(kbase + n * D + 8 * e);
            if constexpr (!SHARED_KV) pv[uu][rr] = ldg16(vbase + n * D + 8 * e);
          } else {
            pk[uu][rr] = u32x4{0u, 0u, 0u, 0u};
            if constexpr (!SHARED_KV) pv[uu][rr] = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int uu = 0; uu < UPT; ++uu) {
      const int u = tid + uu * NT;
      if (U % NT == 0 || u < U) {
        const int pr = u / G8, e = u - pr * G8;
        const int j0 = 2 * pr;
        *reinterpret_cast<u32x4*>(&ks[buf][j0 * KP + 8 * e]) = pk[uu][0];
        *reinterpret_cast<u32x4*>(&ks[buf][(j0 + 1) * KP + 8 * e]) = pk[uu][1];
        const u32x4 w0 = SHARED_KV ? pk[uu][0] : pv[uu][0];
        const u32x4 w1 = SHARED_KV ? pk[uu][1] : pv[uu][1];
        const int col = (j0 & ~31) + key_slot(j0 & 31);   // even; j0+1 lands at col+1
        unsigned int* vrow = reinterpret_cast<unsigned int*>(&vt[buf][0]);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const unsigned int lo = (w0[qq] & 0xFFFFu) | (w1[qq] << 16);
          const unsigned int hi = (w0[qq] >> 16) | (w1[qq] & 0xFFFF0000u);
          const int d = 8 * e + 2 * qq;
          vrow[(d * VP + col) >> 1] = lo;
          vrow[((d + 1) * VP + col) >> 1] = hi;
        }
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int tvalid = (int)min((int64_t)kTJ, n1 - (n0 + (int64_t)t * kTJ));
#pragma unroll
    for (int half = 0; half < kTJ / 32; ++half) {
      const int kvalid = min(32, tvalid - 32 * half);
      if (kvalid > 0) {
        V8 kop[2][KD];
        V8 vop[NDB];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int kd = 0; kd < KD; ++kd) {
            const int d0 = 32 * kd + 8 * g;
            if (d0 < D)
              kop[jb][kd] = *reinterpret_cast<const V8*>(
                  &ks[buf][(32 * half + 16 * jb + r) * KP + d0]);
            else
              kop[jb][kd] = bitcast_u4<V8>(u32x4{0u, 0u, 0u, 0u});
          }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          vop[db] = *reinterpret_cast<const V8*>(&vt[buf][(16 * db + r) * VP + 32 * half + 8 * g]);
        st.step(kop, vop, kvalid, g);
      }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // partials of this chunk
  const int64_t base = ((int64_t)bh * a.nchunks + chunk) * a.Mpad;
#pragma unroll
  for (int cb = 0; cb < kNC; ++cb) {
    const int col = wave * 16 * kNC + cb * 16 + r;
    const float lt = st.row_sum(cb);
    if (g == 0) {
      a.part_m[base + col] = -st.negm[cb][0];
      a.part_l[base + col] = lt;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d0 = 16 * db + 4 * g;
      if (d0 < D) {
        float* dst = a.part_o + (base + col) * D + d0;
        *reinterpret_cast<f32x4*>(dst) = st.o[db][cb];
      }
    }
  }
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
    q[d] = qb[(int64_t)m * D + d];
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

template <typename T, int D>
hipError_t launch_mfma(const EncodeParams& p, hipStream_t s) {
  const int nw = encode_waves(p.M);
  const dim3 grid((unsigned)(p.B * p.H * p.nchunks));
  const bool shared_kv = (p.k == p.v);
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

int encode_waves(int M) {
  const int w = (M + 16 * kNC - 1) / (16 * kNC);
  return w <= 1 ? 1 : w <= 2 ? 2 : w <= 4 ? 4 : 8;
}

int latent_pad(int M, int dtype) {
  // fp32 path: one thread per latent row in blocks of 64; matrix-core path:
  // 64 latents per wave and a power-of-two wave count.
  if (dtype == kF32) return ((M + 63) / 64) * 64;
  return encode_waves(M) * 16 * kNC;
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
