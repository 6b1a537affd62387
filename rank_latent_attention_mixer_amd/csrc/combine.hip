// Merge of the split-encoder partials and the operand copies for the next
// step.
//
// merged(m, d) = sum_c 2^(m_c - m*) O_c[m][d] / sum_c 2^(m_c - m*) l_c[m],
//   m* = max_c m_c
// is the log-sum-exp reduction of issue #2024, "Multi-GPU context
// parallelism" (exact token-sharded encoder), applied across token chunks.
//
// Query mode (after the synthesis): q = q_fixed + sigma(g_h) * merged, the
// "Fixed reference and gate" update of issue #2024 "Changes from v1 to v2";
// sigma = 0 (closed gate) gives q = q_fixed without reading the partials.
// The routing query is written once, prescaled by scale*log2(e) and rounded
// to the operand dtype, in natural [m][d] layout; it serves both as the
// register-side operand of the encoder and as the key operand of the decoder.
//
// Value mode (after the encode): z = merged (or a caller-given z), written
// as the decoder's value operand: rows d permuted so that every lane ends up
// owning contiguous output columns, latents in key-slot order.
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

__device__ __forceinline__ float merged_value(const CombineParams& a, int set, int m, int d) {
  const int64_t base = (int64_t)set * a.nchunks * a.Mpad + m;
  float mstar = -__builtin_inff();
  for (int c = 0; c < a.nchunks; ++c) mstar = fmaxf(mstar, a.part_m[base + (int64_t)c * a.Mpad]);
  float L = 0.f, O = 0.f;
  for (int c = 0; c < a.nchunks; ++c) {
    const int64_t i = base + (int64_t)c * a.Mpad;
    const float w = exp2f(a.part_m[i] - mstar);
    L = fmaf(w, a.part_l[i], L);
    O = fmaf(w, a.part_o[i * a.D + d], O);
  }
  return O / L;
}


__global__ __launch_bounds__(256) void combine_kernel(CombineParams a) {
  const int set = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int width = a.out_kind == kOutValueT ? a.DV : a.D;
  if (idx >= (int64_t)a.Mpad * width) return;
  const int m = (int)(idx / width), d = (int)(idx - (int64_t)m * width);
  const int h = set % a.H;
  const bool live = (m < a.M) && (d < a.D);

  float val = 0.f;
  if (a.mode == kModeQuery) {
    if (live) {
      const int b = set / a.H;
      const float fx = a.fixed ? load_as_float(a.fixed, b * a.fixed_b_stride +
                                                            ((int64_t)h * a.M + m) * a.D + d,
                                               a.fixed_dtype)
                               : 0.f;
      const float sg = (a.force_fixed || a.gate == nullptr) ? (a.force_fixed ? 0.f : 1.f)
                                                            : gate_sigma(a.gate[h]);
      val = (sg == 0.f || a.nchunks == 0) ? fx : fmaf(sg, merged_value(a, set, m, d), fx);
      val *= a.cscale;
    }
  } else {
    if (live) {
      val = a.nchunks == 0 ? a.z_in[((int64_t)set * a.M + m) * a.D + d]
                           : merged_value(a, set, m, d);
      if (a.z_out) a.z_out[((int64_t)set * a.M + m) * a.D + d] = val;
    }
  }
  if (a.out_kind == kOutValueT) {
    const int row = (d & ~31) + value_row(d & 31);  // padded columns map to zero rows
    const int col = (m & ~31) + key_slot(m & 31);
    store_from_float(a.out, ((int64_t)set * a.DV + row) * a.Mpad + col, a.out_dtype, val);
  } else {
    store_from_float(a.out, ((int64_t)set * a.Mpad + m) * a.D + d,
                     a.out_kind == kOutNatural32 ? (int)kF32 : a.out_dtype, val);
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  const int width = p.out_kind == kOutValueT ? p.DV : p.D;
  const int64_t n = (int64_t)p.Mpad * width;
  const dim3 grid((unsigned)((n + 255) / 256), (unsigned)p.nsets);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace flarepp
