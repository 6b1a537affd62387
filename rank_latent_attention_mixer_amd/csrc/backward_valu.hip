// Backward pass on the VALU: fp32 inputs at every D, and bf16 / fp16 at
// D = 8 (below the matrix-core contraction length of 16).  The gradients are
// the chain rule through the forward, one attention at a time
// (FLARE.py README, "FLARE++" and "FLARE" listings; for O = softmax_rows(
// s Q K^T) V with output gradient dO: dV = A^T dO, dS = A * (dO V^T -
// rowsum(dO * O)), dQ = s dS K, dK = s dS^T Q), with the saved base-2
// log-sum-exp rows of the training forward giving every normalised weight
// as A = 2^(S' - lse), S' = c q.k, c = s log2(e).
//
// Two kernels do the work, as the forward's fp32 kernels do: a latent pass
// (one thread per latent row, token tiles staged in LDS, per-chunk partial
// sums over the tokens) and a token pass (one thread per token, latent
// tiles staged in LDS).  All arithmetic is fp32; every reduction runs in a
// fixed order, so results are deterministic.  The latent operand is c q
// rounded to the input dtype, as the forward's matrix-core operand is, so
// the recomputed weights match the saved normalisers.
#include "backward.hpp"
#include "flarepp_device.hpp"

namespace flarepp {

namespace {

template <int V>
struct IntD {
  static constexpr int value = V;
};
template <typename T>
struct TypeTag {
  using type = T;
};

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  return (float)reinterpret_cast<const T*>(p)[i];
}

// c q, rounded to the operand dtype where the forward rounds it
__device__ __forceinline__ float scaled_operand(float q, float c, int dtype) {
  const float x = c * q;
  if (dtype == kBF16) return (float)(__bf16)x;
  if (dtype == kF16) return (float)(_Float16)x;
  return x;
}

__device__ __forceinline__ float lat_elem(const void* p, int dt, int64_t i) {
  if (dt == kF32) return reinterpret_cast<const float*>(p)[i];
  if (dt == kBF16) return (float)reinterpret_cast<const __bf16*>(p)[i];
  return (float)reinterpret_cast<const _Float16*>(p)[i];
}

__device__ __forceinline__ bool head_closed(const float* gate, int h) {
  return gate != nullptr && gate_sigma(gate[h]) == 0.f;
}

// -Delta2 = -(dy . y) per token row.
template <typename T, int D>
__global__ __launch_bounds__(256) void valu_negd_kernel(const void* dy, const void* y, float* out,
                                                        int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) acc = fmaf(ld<T>(dy, r * D + d), ld<T>(y, r * D + d), acc);
  out[r] = -acc;
}

// Latent pass.  Per latent m of set (b, h) and token chunk:
//   Dec: A = 2^(S' - lse2_n), G = dy_n.z_m - Delta2_n:  Y += A G k_n, X += A dy_n
//   Enc: A = 2^(S' - lse1_m), G = dz_m.v_n - Delta1_m:  Y += A G k_n
//   Syn: A = 2^(S0' - lse0_m), G = dqd_m.w_n - Delta0_m (w = k0 or v0): Y += A G k0_n
// and writes s Y (and X) as the chunk's partials.
template <typename T, int D>
__global__ __launch_bounds__(64) void valu_lat_kernel(BwdValuLatParams a) {
  constexpr int TJ = 32;
  __shared__ float tk[TJ][D];
  __shared__ float tg[TJ][D];
  __shared__ float tstat[TJ][2];
  const int m = blockIdx.x * 64 + threadIdx.x;
  const int chunk = blockIdx.y;
  const int bh = blockIdx.z;
  const int b = bh / a.H, h = bh - b * a.H;
  const bool live = m < a.M;
  const int64_t pbase = (((int64_t)bh * a.nchunks + chunk) * a.M + (live ? m : 0)) * D;
  if (a.mode == kBwdLatSyn && head_closed(a.gate, h)) {
    if (live) {
#pragma unroll
      for (int d = 0; d < D; ++d) a.part_y[pbase + d] = 0.f;
    }
    return;
  }
  const int64_t n0 = (int64_t)chunk * a.chunk_tokens;
  const int64_t n1 = min(a.N, n0 + a.chunk_tokens);
  float q[D], g[D], y[D], x[D];
  float lse_m = 0.f, negd_m = 0.f;
  const int mm = live ? m : 0;
  const int64_t qoff = b * a.q_b_stride + h * a.q_h_stride + (int64_t)mm * D;
  const int64_t goff = ((int64_t)bh * a.M + mm) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = scaled_operand(lat_elem(a.qlat, a.qlat_dtype, qoff + d), a.c, a.round_dtype);
    g[d] = a.glat[goff + d];
    y[d] = 0.f;
    x[d] = 0.f;
  }
  if (a.mode != kBwdLatDec) {
    lse_m = a.lse_lat[(int64_t)bh * a.M + mm];
    negd_m = a.negd_lat[(int64_t)bh * a.M + mm];
  }
  const int64_t tbase = (int64_t)bh * a.N;
  for (int64_t t0 = n0; t0 < n1; t0 += TJ) {
    const int tv = (int)min((int64_t)TJ, n1 - t0);
    for (int e = threadIdx.x; e < TJ * D; e += 64) {
      const int j = e / D, d = e - j * D;
      const bool in = j < tv;
      tk[j][d] = in ? ld<T>(a.tk, (tbase + t0 + j) * D + d) : 0.f;
      tg[j][d] = in ? ld<T>(a.tg, (tbase + t0 + j) * D + d) : 0.f;
    }
    if (a.mode == kBwdLatDec && threadIdx.x < TJ) {
      const int j = threadIdx.x;
      tstat[j][0] = j < tv ? a.lse_tok[tbase + t0 + j] : 0.f;
      tstat[j][1] = j < tv ? a.negd_tok[tbase + t0 + j] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < tv; ++j) {
      float sc = 0.f, gd = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        sc = fmaf(q[d], tk[j][d], sc);
        gd = fmaf(g[d], tg[j][d], gd);
      }
      float A, G;
      if (a.mode == kBwdLatDec) {
        A = exp2f(sc - tstat[j][0]);
        G = gd + tstat[j][1];
#pragma unroll
        for (int d = 0; d < D; ++d) x[d] = fmaf(A, tg[j][d], x[d]);
      } else {
        A = exp2f(sc - lse_m);
        G = gd + negd_m;
      }
      const float t = A * G;
#pragma unroll
      for (int d = 0; d < D; ++d) y[d] = fmaf(t, tk[j][d], y[d]);
    }
    __syncthreads();
  }
  if (!live) return;
#pragma unroll
  for (int d = 0; d < D; ++d) a.part_y[pbase + d] = a.s * y[d];
  if (a.mode == kBwdLatDec) {
#pragma unroll
    for (int d = 0; d < D; ++d) a.part_x[pbase + d] = x[d];
  }
}

// Token pass.  Per token n of set (b, h), over every latent m:
//   Flare: A2 = 2^(S' - lse2_n), A1 = 2^(S' - lse1_m),
//          dk_n = s/c sum_m (A2 (dy_n.z_m - Delta2_n) + A1 (dz_m.v_n - Delta1_m)) (c q_m),
//          dv_n = sum_m A1 dz_m
//   Syn:   A0 = 2^(S0' - lse0_m), key part s/c sum_m A0 (dqd_m.w_n - Delta0_m) (c q0_m),
//          value part sum_m A0 dqd_m (added to the key part when w = k0)
template <typename T, int D>
__global__ __launch_bounds__(256) void valu_tok_kernel(BwdValuTokParams a) {
  constexpr int TM = 32;
  __shared__ float lq[TM][D];
  __shared__ float lz[TM][D];
  __shared__ float ldz[TM][D];
  __shared__ float lst[TM][2];
  const int64_t bpb = (a.N + 255) / 256;
  const int bh = (int)(blockIdx.x / bpb);
  const int b = bh / a.H, h = bh - b * a.H;
  const int64_t n = ((int64_t)blockIdx.x - (int64_t)bh * bpb) * 256 + threadIdx.x;
  const bool live = n < a.N;
  const int64_t row = ((int64_t)bh * a.N + (live ? n : 0)) * D;
  if (a.mode == kBwdTokSyn && head_closed(a.gate, h)) {
    if (live) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        a.out_k[row + d] = 0.f;
        if (a.out_v) a.out_v[row + d] = 0.f;
      }
    }
    return;
  }
  const bool flare = a.mode == kBwdTokFlare;
  float k[D], dyv[D], w[D], ak[D], av[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    k[d] = ld<T>(a.tk, row + d);
    dyv[d] = flare ? ld<T>(a.tdy, row + d) : 0.f;
    w[d] = ld<T>(a.tw, row + d);
    ak[d] = 0.f;
    av[d] = 0.f;
  }
  const float lse2 = flare ? a.lse_tok[(int64_t)bh * a.N + (live ? n : 0)] : 0.f;
  const float negd2 = flare ? a.negd_tok[(int64_t)bh * a.N + (live ? n : 0)] : 0.f;
  const int64_t qset = b * a.q_b_stride + h * a.q_h_stride;
  const int64_t lset = (int64_t)bh * a.M;
  for (int m0 = 0; m0 < a.M; m0 += TM) {
    const int mv = min(TM, a.M - m0);
    for (int e = threadIdx.x; e < TM * D; e += 256) {
      const int j = e / D, d = e - j * D;
      const bool in = j < mv;
      lq[j][d] = in ? scaled_operand(lat_elem(a.qlat, a.qlat_dtype, qset + (int64_t)(m0 + j) * D + d),
                                     a.c, a.round_dtype)
                    : 0.f;
      lz[j][d] = (in && flare) ? a.lat_z[(lset + m0 + j) * D + d] : 0.f;
      ldz[j][d] = in ? a.lat_g[(lset + m0 + j) * D + d] : 0.f;
    }
    if (threadIdx.x < TM) {
      const int j = threadIdx.x;
      lst[j][0] = j < mv ? a.lse_lat[lset + m0 + j] : 0.f;
      lst[j][1] = j < mv ? a.negd_lat[lset + m0 + j] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < mv; ++j) {
      float sc = 0.f, g1 = 0.f, g2 = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        sc = fmaf(lq[j][d], k[d], sc);
        g1 = fmaf(ldz[j][d], w[d], g1);
        if (flare) g2 = fmaf(dyv[d], lz[j][d], g2);
      }
      const float A1 = exp2f(sc - lst[j][0]);
      float t = A1 * (g1 + lst[j][1]);
      if (flare) t = fmaf(exp2f(sc - lse2), g2 + negd2, t);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        ak[d] = fmaf(t, lq[j][d], ak[d]);
        av[d] = fmaf(A1, ldz[j][d], av[d]);
      }
    }
    __syncthreads();
  }
  if (!live) return;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float key = a.s_over_c * ak[d];
    if (a.out_v) {
      a.out_k[row + d] = key;
      a.out_v[row + d] = av[d];
    } else {
      a.out_k[row + d] = key + av[d];
    }
  }
}

// Chunk sums: dst[set][m][:] (+)= sum_c part[set][c][m][:] in chunk order;
// with w and negd, also -Delta = -(dst . w) per latent row.
template <int D>
__global__ __launch_bounds__(64) void valu_sum_kernel(const float* part, int nchunks, int M,
                                                      int sets, float* dst, int accumulate,
                                                      const float* w, float* negd) {
  const int64_t r = (int64_t)blockIdx.x * 64 + threadIdx.x;  // (set, m)
  if (r >= (int64_t)sets * M) return;
  const int64_t set = r / M, m = r - set * M;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = accumulate ? dst[r * D + d] : 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const float* p = part + ((set * nchunks + c) * M + m) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] += p[d];
  }
  float dot = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    dst[r * D + d] = acc[d];
    if (w) dot = fmaf(acc[d], w[r * D + d], dot);
  }
  if (negd) negd[r] = -dot;
}

// Latent gradient summed over the batch: out[h][m][d] = sum_b src[b,h][m][d].
// FLARE++ (sigma non-null): also dqd[b,h] = sigma_h src[b,h] and -Delta0 =
// -(dqd . qd) per latent; simplified (sigma null, dqd non-null): dqd = src.
__global__ __launch_bounds__(256) void valu_batch_sum_kernel(const float* src, int B, int H, int M,
                                                             int D, float* out, const float* gate,
                                                             float* dqd) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (h, m, d)
  const int64_t per = (int64_t)M * D;
  if (i >= (int64_t)H * per) return;
  const int h = (int)(i / per);
  const int64_t md = i - (int64_t)h * per;
  const float sg = gate ? gate_sigma(gate[h]) : 1.f;
  float acc = 0.f;
  for (int b = 0; b < B; ++b) {
    const float v = src[((int64_t)b * H + h) * per + md];
    acc += v;
    if (dqd) dqd[((int64_t)b * H + h) * per + md] = sg * v;
  }
  if (out) out[i] = acc;
}

// -Delta0 = -(dqd . qd) per (b, h, m).
__global__ __launch_bounds__(256) void valu_negd_rows_kernel(const float* a, const float* w,
                                                             int64_t rows, int D, float* out) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float dot = 0.f;
  for (int d = 0; d < D; ++d) dot = fmaf(a[r * D + d], w[r * D + d], dot);
  out[r] = -dot;
}

// dgate_h = sigma'(g_h) sum_{b,m,d} dq[b,h,m,d] qd[b,h,m,d], one workgroup
// per head, fixed-order tree over 256 threads.
__global__ __launch_bounds__(256) void valu_gate_kernel(const float* dq, const float* qd, int B,
                                                        int H, int M, int D, const float* gate,
                                                        float* dgate) {
  __shared__ float red[256];
  const int h = blockIdx.x;
  const int64_t per = (int64_t)M * D;
  float acc = 0.f;
  for (int b = 0; b < B; ++b) {
    const int64_t base = ((int64_t)b * H + h) * per;
    for (int64_t i = threadIdx.x; i < per; i += 256) acc = fmaf(dq[base + i], qd[base + i], acc);
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float sg = gate_sigma(gate[h]);
    const float dsg = sg * (1.f - sg);
    dgate[h] = dsg == 0.f ? 0.f : dsg * red[0];
  }
}

template <typename T, int D>
hipError_t lat_t(const BwdValuLatParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((p.M + 63) / 64), (unsigned)p.nchunks, (unsigned)(p.B * p.H));
  hipLaunchKernelGGL((valu_lat_kernel<T, D>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t tok_t(const BwdValuTokParams& p, hipStream_t s) {
  const int64_t blocks = (p.N + 255) / 256 * p.B * p.H;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((valu_tok_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}
template <typename T, int D>
hipError_t negd_t(const void* dy, const void* y, float* out, int64_t rows, hipStream_t s) {
  const int64_t blocks = (rows + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((valu_negd_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, dy, y,
                     out, rows);
  return hipGetLastError();
}

template <typename F>
hipError_t by_type_d(int dtype, int D, F&& f) {
  auto pick_d = [&](auto tag) -> hipError_t {
    using T = typename decltype(tag)::type;
    switch (D) {
      case 8: return f(T{}, IntD<8>{});
      case 16: return f(T{}, IntD<16>{});
      case 32: return f(T{}, IntD<32>{});
      case 64: return f(T{}, IntD<64>{});
      default: return hipErrorInvalidValue;
    }
  };
  if (dtype == kF32) return pick_d(TypeTag<float>{});
  if (dtype == kBF16) return pick_d(TypeTag<__bf16>{});
  if (dtype == kF16) return pick_d(TypeTag<_Float16>{});
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_valu_lat(int dtype, int D, const BwdValuLatParams& p, hipStream_t s) {
  return by_type_d(dtype, D, [&](auto t, auto d) -> hipError_t {
    return lat_t<decltype(t), decltype(d)::value>(p, s);
  });
}

hipError_t launch_bwd_valu_tok(int dtype, int D, const BwdValuTokParams& p, hipStream_t s) {
  return by_type_d(dtype, D, [&](auto t, auto d) -> hipError_t {
    return tok_t<decltype(t), decltype(d)::value>(p, s);
  });
}

hipError_t launch_bwd_valu_negd(int dtype, int D, const void* dy, const void* y, float* out,
                                int64_t rows, hipStream_t s) {
  return by_type_d(dtype, D, [&](auto t, auto d) -> hipError_t {
    return negd_t<decltype(t), decltype(d)::value>(dy, y, out, rows, s);
  });
}

hipError_t launch_bwd_valu_sum(int D, const float* part, int nchunks, int M, int sets, float* dst,
                               int accumulate, const float* w, float* negd, hipStream_t s) {
  const int64_t rows = (int64_t)sets * M;
  const dim3 grid((unsigned)((rows + 63) / 64));
  switch (D) {
    case 8: hipLaunchKernelGGL(valu_sum_kernel<8>, grid, dim3(64), 0, s, part, nchunks, M, sets, dst, accumulate, w, negd); break;
    case 16: hipLaunchKernelGGL(valu_sum_kernel<16>, grid, dim3(64), 0, s, part, nchunks, M, sets, dst, accumulate, w, negd); break;
    case 32: hipLaunchKernelGGL(valu_sum_kernel<32>, grid, dim3(64), 0, s, part, nchunks, M, sets, dst, accumulate, w, negd); break;
    case 64: hipLaunchKernelGGL(valu_sum_kernel<64>, grid, dim3(64), 0, s, part, nchunks, M, sets, dst, accumulate, w, negd); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_valu_batch_sum(const float* src, int B, int H, int M, int D, float* out,
                                     const float* gate, float* dqd, hipStream_t s) {
  const int64_t n = (int64_t)H * M * D;
  hipLaunchKernelGGL(valu_batch_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     src, B, H, M, D, out, gate, dqd);
  return hipGetLastError();
}

hipError_t launch_bwd_valu_negd_rows(const float* a, const float* w, int64_t rows, int D,
                                     float* out, hipStream_t s) {
  hipLaunchKernelGGL(valu_negd_rows_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                     s, a, w, rows, D, out);
  return hipGetLastError();
}

hipError_t launch_bwd_valu_gate(const float* dq, const float* qd, int B, int H, int M, int D,
                                const float* gate, float* dgate, hipStream_t s) {
  hipLaunchKernelGGL(valu_gate_kernel, dim3((unsigned)H), dim3(256), 0, s, dq, qd, B, H, M, D,
                     gate, dgate);
  return hipGetLastError();
}

}  // namespace flarepp
