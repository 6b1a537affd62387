// Device-side building blocks shared by the FLARE++ kernels (gfx950 only).
//
// Matrix-core tile used throughout: v_mfma_f32_32x32x16_{bf16,f16}.
// For D[32x32] += A[32x16] * B[16x32], lane l of the 64-wide wave (h = l/32)
// supplies
//   A[l % 32][8h .. 8h+7]     (8 consecutive k of one row)
//   B[8h .. 8h+7][l % 32]     (8 consecutive k of one column)
// and receives the 16 values D[8a + 4h + i][l % 32], v = 4a + i (a, i = 0..3).
// (The 32x32 shape is used rather than 16x16x32 because it leaves the VALU
// far more room to run the softmax exponentials alongside the matrix core.)
//
// Attention is evaluated "transposed": for query columns r (held in
// registers) and keys j (streamed), the score tile is S^T[j][r] =
// K[j] . Q[r], so each lane owns one query column and 16 keys.  Those 16
// fp32 scores, after exp and packing, are exactly the k-values that lane
// must supply as the B operand of the two K=16 steps of the P.V product
// O^T[d][r] += V^T[d][j] P^T[j][r].  The price is that V must be supplied
// transposed (rows d, k = keys) in the key order the score layout implies:
// within a 32-key group, operand slot s = 16kk + 8h + 4a + i holds key
// j = 16kk + 8a + 4h + i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flarepp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

// log2(e): scores are carried in the base-2 domain so that exp is one
// v_exp_f32.  The caller folds scale * log2(e) into the latent operand.
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Pack8;
template <> struct Pack8<__bf16> { typedef bf16x8 type; typedef bf16x2 pair; };
template <> struct Pack8<_Float16> { typedef f16x8 type; typedef f16x2 pair; };

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x32: lane l supplies A[l%16][8(l/16) ..+7] and
// B[8(l/16) ..+7][l%16] and receives D[4(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <typename V>
__device__ __forceinline__ V bitcast_u4(u32x4 x) {
  return __builtin_bit_cast(V, x);
}
template <typename V>
__device__ __forceinline__ u32x4 to_u4(V x) {
  return __builtin_bit_cast(u32x4, x);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// 16 bytes per lane from global memory straight into LDS (no registers):
// lane i's data lands at lds_base + 16*i, lds_base being wave-uniform.
// The builtin exists only in the device pass; in the host pass of the
// single-source compile its presence would drop the kernel's launch stub.
__device__ __forceinline__ void global_to_lds16(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   0);
#endif
}
// The same with the non-temporal hint (data read once: it is not kept in
// the caches at the expense of data that is read again).
__device__ __forceinline__ void global_to_lds16_nt(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   2);
#endif
}

// Convert 8 fp32 to a packed 8-element operand (round to nearest even).
template <typename T>
__device__ __forceinline__ typename Pack8<T>::type pack8(float a0, float a1, float a2, float a3,
                                                        float a4, float a5, float a6, float a7) {
  typename Pack8<T>::type r;
  r[0] = (T)a0; r[1] = (T)a1; r[2] = (T)a2; r[3] = (T)a3;
  r[4] = (T)a4; r[5] = (T)a5; r[6] = (T)a6; r[7] = (T)a7;
  return r;
}

// Eight probabilities packed as a matrix-core operand.  bf16 keeps the upper
// half of each fp32 (truncation, one v_perm_b32 per pair): only the spread
// of the per-element rounding errors reaches the normalised result -- a
// common factor cancels between numerator and row sum -- and that spread is
// one unit in the last place for truncation as for round-to-nearest; an
// infinite probability stays infinite.  fp16 rounds to nearest even
// (v_cvt_pk_f16_f32), so a probability beyond the fp16 range becomes
// infinite and the sweep's range check sees it (a saturating conversion
// would hide it).
template <typename T>
__device__ __forceinline__ typename Pack8<T>::type pack_probs(const float (&e)[8]);
template <>
__device__ __forceinline__ bf16x8 pack_probs<__bf16>(const float (&e)[8]) {
  u32x4 w;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    w[t] = __builtin_amdgcn_perm(__builtin_bit_cast(unsigned, e[2 * t + 1]),
                                 __builtin_bit_cast(unsigned, e[2 * t]), 0x07060302u);
  return __builtin_bit_cast(bf16x8, w);
}
template <>
__device__ __forceinline__ f16x8 pack_probs<_Float16>(const float (&e)[8]) {
  return pack8<_Float16>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
}

// Operand slot of key j within a 32-key group (see header comment).
__host__ __device__ __forceinline__ int key_slot(int j) {
  const int kk = j >> 4, a = (j >> 3) & 1, h = (j >> 2) & 1, i = j & 3;
  return 16 * kk + 8 * h + 4 * a + i;
}

// Row of a 32-row value block that must hold output column d (0..31) so
// that the lane half h = d/16 receives columns 16h .. 16h+15 in order:
// accumulator row 8a + 4h + i is value v = 4a + i of lane half h.
__host__ __device__ __forceinline__ int value_row(int d) {
  const int h = d >> 4, a = (d >> 2) & 3, i = d & 3;
  return 8 * a + 4 * h + i;
}

// Eight consecutive latent elements as a scaled operand: (T)(s * x), each
// rounded to nearest even -- the same bits as an operand copy formed
// elementwise in fp32 beforehand.
template <typename T>
__device__ __forceinline__ u32x4 scaled8(const T* p, float s) {
  const u32x4 raw = ldg16(p);
  typename Pack8<T>::type x = bitcast_u4<typename Pack8<T>::type>(raw), y;
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (T)(s * (float)x[i]);
  return to_u4(y);
}

// Logistic gate in fp32; -inf -> 0, +inf -> 1.
__device__ __forceinline__ float gate_sigma(float g) {
  return 1.0f / (1.0f + expf(-g));
}

}  // namespace flarepp
