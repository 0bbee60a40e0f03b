// Device-side helpers shared by the gfx950 kernels: element types, 16-byte
// vectors, bf16 conversion, and the two MFMA steps the contractions use.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vit {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16 bytes of elements: 8 bf16 or 4 float.
template <typename T> struct Vec;
template <> struct Vec<bf16> { static constexpr int N = 8; };
template <> struct Vec<float> { static constexpr int N = 4; };

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Unpack / pack 16 bytes as floats.
template <typename T> __device__ __forceinline__ void unpack16(u32x4 v, float* f);
template <> __device__ __forceinline__ void unpack16<bf16>(u32x4 v, float* f) {
  bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)b[i];
}
template <> __device__ __forceinline__ void unpack16<float>(u32x4 v, float* f) {
  f32x4 b = __builtin_bit_cast(f32x4, v);
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = b[i];
}
template <typename T> __device__ __forceinline__ u32x4 pack16(const float* f);
template <> __device__ __forceinline__ u32x4 pack16<bf16>(const float* f) {
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (bf16)f[i];
  return __builtin_bit_cast(u32x4, b);
}
template <> __device__ __forceinline__ u32x4 pack16<float>(const float* f) {
  f32x4 b = {f[0], f[1], f[2], f[3]};
  return __builtin_bit_cast(u32x4, b);
}

// Store 4 consecutive output elements converted from float.
template <typename T> __device__ __forceinline__ void store4(T* p, f32x4 v);
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, f32x4 v) {
  bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, b);
}
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <typename T> __device__ __forceinline__ f32x4 load4(const T* p);
template <> __device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  bf16x4 b = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(p));
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// One 16x16 output-tile MFMA step over a 16-byte-per-lane fragment pair.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, with the 16
// bytes holding contraction chunk g = l / 16. bf16: one 16x16x32 MFMA, chunk
// g = k 8g..8g+7. float: four 16x16x4 MFMAs, MFMA i taking element i of each
// lane's chunk, so k-slot (g, i) is contraction index 4g + i; A and B use the
// same slot order, so the sum is the plain dot product.
// Result: lane l holds D[4*(l/16) + r][l % 16], r = 0..3.
template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KSTEP = 32;
  static __device__ __forceinline__ f32x4 step(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KSTEP = 16;
  static __device__ __forceinline__ f32x4 step(u32x4 a, u32x4 b, f32x4 c) {
    f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[0], fb[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[1], fb[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[2], fb[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[3], fb[3], c, 0, 0, 0);
    return c;
  }
};

// erf-form GELU, 0.5 v (1 + erf(v / sqrt 2)). With z = |v| / sqrt 2, the
// rational approximation of Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (|error| <= 1.5e-7) gives erfc(z) =
// t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z).
// With q = erfc(z) / 2 (the a_i halved), GELU(v) = v (1 - q) for v >= 0 and
// v q for v < 0: the negative tail comes straight from erfc, without the
// cancellation in 1 - erf. Two hardware transcendentals (reciprocal, exp2).
__device__ __forceinline__ float gelu_erf_as(float v) {
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f * 0.70710678118654752f, fabsf(v), 1.0f));
  float poly = __builtin_fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  poly = __builtin_fmaf(t, poly, 0.5f * 1.421413741f);
  poly = __builtin_fmaf(t, poly, 0.5f * -0.284496736f);
  poly = __builtin_fmaf(t, poly, 0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(v * v * (-0.5f * 1.4426950408889634f));  // exp(-z^2)
  // |v| q with q = erfc(|z|)/2 = Phi(-|v|): v - |v| q for v >= 0, -|v| q below,
  // i.e. max(v, 0) - |v| q in one fma
  return __builtin_fmaf(-fabsf(v), (poly * t) * e, fmaxf(v, 0.f));
}

// tanh-approximated GELU, 0.5 v (1 + tanh(u)) with u = sqrt(2/pi)(v + 0.044715 v^3),
// written through 1 + tanh(u) = 2 / (1 + e^(-2u)): v / (1 + 2^(-2u log2 e)).
// One exp2 and one reciprocal (hardware, ~1 ulp each); saturates to v and -0
// for large |u| without overflow trouble (2^+inf -> inf -> reciprocal 0).
__device__ __forceinline__ float gelu_tanh_fast(float v) {
  // -2 u log2(e), the two constants folded into one multiply
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(0.044715f * v, v * v, v) * (0.79788456080286536f * -2.8853900817779268f));
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// Cross-lane reductions without LDS round trips (ds_bpermute):
// row16_*  over each row of 16 lanes with DPP: two quad swaps, then the
//          half-row mirror (lane i <-> 7-i of its 8) and the row mirror
//          (i <-> 15-i) each pair a lane with one of the other half;
// pair16_* over lanes l and l^16, pair32_* over l and l^32, with the gfx950
//          row swaps (v_permlane16_swap / v_permlane32_swap: with both
//          operands x the two results are the two rows' values).
#define VIT_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false))
__device__ __forceinline__ float row16_sum(float x) {
  x += VIT_DPP(x, 0xB1);   // quad_perm [1,0,3,2]
  x += VIT_DPP(x, 0x4E);   // quad_perm [2,3,0,1]
  x += VIT_DPP(x, 0x141);  // row_half_mirror
  x += VIT_DPP(x, 0x140);  // row_mirror
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, VIT_DPP(x, 0xB1));
  x = fmaxf(x, VIT_DPP(x, 0x4E));
  x = fmaxf(x, VIT_DPP(x, 0x141));
  x = fmaxf(x, VIT_DPP(x, 0x140));
  return x;
}
#undef VIT_DPP
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace vit
