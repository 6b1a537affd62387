// Merge of the split-encoder partials and the operand copies for the next
// step.
//
// merged(m, d) = sum_c 2^(m_c - m*) O_c[m][d] / sum_c 2^(m_c - m*) l_c[m],
//   m* = max_c m_c
// is the log-sum-exp reduction of issue #2024, "Multi-GPU context
// parallelism" (exact token-sharded encoder), applied across token chunks.
// It is evaluated as pairwise merges of (m, l, O) states in a fixed order
// (each of four lanes takes every fourth chunk, then a fixed butterfly), so
// the result does not depend on timing.
//
// Query mode (after the synthesis): q = q_fixed + sigma(g_h) * merged, the
// "Fixed reference and gate" update of issue #2024 "Changes from v1 to v2";
// sigma = 0 (closed gate) gives q = q_fixed without reading the partials.
// The routing query is written once, prescaled by scale*log2(e) and rounded
// to the operand dtype, in natural [m][d] layout; it serves both as the
// register-side operand of the encoder and as the key operand of the decoder.
//
// Value mode (after the encode): z = merged (or a caller-given z), written
// as the decoder's value operand in natural [m][d] layout, rounded to the
// operand dtype (the decoder permutes it into its matrix-core layout as it
// fills its LDS).
#include "flarepp_device.hpp"
#include "kernels.hpp"

namespace flarepp {

namespace {

__device__ __forceinline__ float load_as_float(const void* p, int64_t i, int dtype) {
  if (dtype == kBF16) return (float)reinterpret_cast<const __bf16*>(p)[i];
  if (dtype == kF16) return (float)reinterpret_cast<const _Float16*>(p)[i];
  return reinterpret_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_from_float(void* p, int64_t i, int dtype, float x) {
  if (dtype == kBF16) reinterpret_cast<__bf16*>(p)[i] = (__bf16)x;
  else if (dtype == kF16) reinterpret_cast<_Float16*>(p)[i] = (_Float16)x;
  else reinterpret_cast<float*>(p)[i] = x;
}

// Running log-sum-exp state of one (latent, 4 columns) slot.
struct Lse {
  float m, l;
  f32x4 o;
};

// a (+) b: both rescaled to the larger reference; an empty side (m = -inf)
// contributes nothing.
__device__ __forceinline__ Lse lse_merge(const Lse& a, const Lse& b) {
  const float mn = fmaxf(a.m, b.m);
  const float wa = a.m == -__builtin_inff() ? 0.f : exp2f(a.m - mn);
  const float wb = b.m == -__builtin_inff() ? 0.f : exp2f(b.m - mn);
  Lse r;
  r.m = mn;
  r.l = a.l * wa + b.l * wb;
  r.o = a.o * wa + b.o * wb;
  return r;
}

// Base-2 log-sum-exp of a merged state: m + log2(l).
__device__ __forceinline__ float lse_state_base2(float m, float l) { return m + log2f(l); }

// One thread per (latent set, latent m, 4 output columns, lane of the
// slot): each of the L lanes of a slot (L = 1, 2, 4 or 8, fixed by the chunk
// count) merges every L-th chunk, then the lanes combine in a fixed
// butterfly and the first lane writes.
__global__ __launch_bounds__(256) void combine_kernel(CombineParams a) {
  const int set = blockIdx.x;  // sets along x: their count may pass the y limit
  const int W4 = a.D / 4;
  const int lg = a.lanes_log2, L = 1 << lg;
  const int64_t t = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  const int sub = (int)(t & (L - 1));
  const int64_t slot = t >> lg;
  const bool in_range = slot < (int64_t)a.Mpad * W4;  // all lanes stay for the shuffles
  const int m = in_range ? (int)(slot / W4) : 0;
  const int d0 = in_range ? 4 * (int)(slot - (int64_t)m * W4) : 0;
  const int h = set % a.H;
  const bool live = in_range && m < a.M;  // D is a multiple of 4

  float sg = 1.f;
  bool use_parts = a.nchunks > 0;
  if (a.mode == kModeQuery) {
    sg = (a.force_fixed || a.gate == nullptr) ? (a.force_fixed ? 0.f : 1.f) : gate_sigma(a.gate[h]);
    use_parts = use_parts && sg != 0.f;
  }

  f32x4 merged = {0.f, 0.f, 0.f, 0.f};
  float lse_m = 0.f, lse_l = 1.f;
  if (use_parts) {  // uniform over the grid
    Lse st{-__builtin_inff(), 0.f, {0.f, 0.f, 0.f, 0.f}};
    if (live) {
      const int64_t base = (int64_t)set * a.nchunks * a.Mpad + m;
#pragma unroll 4
      for (int c = sub; c < a.nchunks; c += L) {
        const int64_t i = base + (int64_t)c * a.Mpad;
        Lse x;
        x.m = a.part_m[i];
        x.l = a.part_l[i];
        x.o = *reinterpret_cast<const f32x4*>(a.part_o + i * a.D + d0);
        st = lse_merge(st, x);
      }
    }
    for (int x = 1; x < L; x <<= 1) {  // L is uniform over the grid
      Lse o;
      o.m = __shfl_xor(st.m, x);
      o.l = __shfl_xor(st.l, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) o.o[e] = __shfl_xor(st.o[e], x);
      st = lse_merge(st, o);
    }
    merged = st.o / st.l;
    lse_m = st.m;
    lse_l = st.l;
  }
  if (!in_range || sub != 0) return;

  float val[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    const int64_t ri = ((int64_t)set * a.M + m) * a.D + d0;  // natural [sets][M][D]
    if (a.lse_out && d0 == 0)
      a.lse_out[(int64_t)set * a.M + m] = use_parts ? lse_state_base2(lse_m, lse_l) : 0.f;
    if (a.mode == kModeQuery) {
      const int b = set / a.H;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fx =
            a.fixed ? load_as_float(a.fixed, b * a.fixed_b_stride + ((int64_t)h * a.M + m) * a.D + d0 + e,
                                    a.fixed_dtype)
                    : 0.f;
        const float qv = use_parts ? fmaf(sg, merged[e], fx) : fx;
        if (a.q_out) a.q_out[ri + e] = qv;
        if (a.dyn_out) a.dyn_out[ri + e] = use_parts ? merged[e] : 0.f;
        val[e] = qv * a.cscale;
      }
    } else {
      const int64_t zi = ((int64_t)set * a.M + m) * a.D + d0;
      if (a.nchunks == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = a.z_in[zi + e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = merged[e];
      }
      if (a.z_out) {  // caller memory: element stores, no alignment assumed
#pragma unroll
        for (int e = 0; e < 4; ++e) a.z_out[zi + e] = val[e];
      }
    }
  }
  const int od = a.out_kind == kOutNatural32 ? (int)kF32 : a.out_dtype;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    store_from_float(a.out, ((int64_t)set * a.Mpad + m) * a.D + d0 + e, od, val[e]);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  // lanes per slot: each merges at most eight chunks, up to eight lanes
  // (same box: with 4 chunks a lane beat four lanes of one chunk by 40%,
  // and with 32 chunks four lanes of 8 beat eight lanes of 4 by 8%)
  CombineParams c = p;
  c.lanes_log2 = 0;
  while (c.lanes_log2 < 3 && (c.nchunks + (1 << c.lanes_log2) - 1) / (1 << c.lanes_log2) > 8)
    ++c.lanes_log2;
  const int64_t n = ((int64_t)c.Mpad * (c.D / 4)) << c.lanes_log2;  // (latent, 4 columns, lane)
  const dim3 grid((unsigned)c.nsets, (unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, c);
  return hipGetLastError();
}

}  // namespace flarepp
