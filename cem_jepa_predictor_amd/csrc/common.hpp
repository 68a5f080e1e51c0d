// Shared device/host definitions of the gfx950 CEM library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cem {

using bf16 = uint16_t;   // storage type: upper 16 bits of an IEEE binary32

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16 v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Two floats -> packed bf16 pair (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}
// Round to nearest, ties to even.
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  return static_cast<bf16>(pack_bf16x2(f, 0.f) & 0xffffu);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
  __device__ static __forceinline__ float to_f32(float v) { return v; }
  __device__ static __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<bf16> {
  __device__ static __forceinline__ float load(const bf16* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void store(bf16* p, float v) { *p = f32_to_bf16(v); }
  __device__ static __forceinline__ float to_f32(bf16 v) { return bf16_to_f32(v); }
  __device__ static __forceinline__ bf16 from_f32(float v) { return f32_to_bf16(v); }
};

// Logical row r of a compact matrix -> physical row of a strided one:
//   phys = (r / group) * stride + offset + r % group.
// Identity: group = INT32_MAX, stride = 0, offset = 0.
struct RowMap {
  int group, stride, offset;
  __host__ __device__ __forceinline__ long long operator()(int r) const {
    return (long long)(r / group) * stride + offset + (r % group);
  }
  static RowMap identity() { return RowMap{0x7fffffff, 0, 0}; }
};

// GEMM epilogue: out[m, n] = act(acc[m, n] + bias[n]) (+ out[m, n] if residual).
// Columns n < split go to c0 (leading dimension ld0), the rest to c1 at
// column n - split (leading dimension ld1).  Output rows go through `rows`.
struct Epilogue {
  const float* bias;   // [N] fp32, nullable
  void* c0;
  void* c1;
  int ld0, ld1, split;
  int gelu;            // 1: exact GELU after the bias
  int residual;        // 1: add the existing output value
  RowMap rows;
};

enum class Act { None, Gelu };

// GELU(x) = x * Phi(x) with Phi from the exact erf (libm erff): fp32 models.
__device__ __forceinline__ float gelu_exact(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// GELU(x) = x * Phi(x) for bf16 models, branch-free.  With h = Phi(-|x|):
// GELU(x) = max(x, 0) - |x| h for either sign.  h = erfc(z) / 2, z = |x| / sqrt(2),
// erfc(z) ~= t (a1 + a2 t + ... + a5 t^4) exp(-z^2), t = 1 / (1 + p z):
// Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26
// (Hastings), |erf error| <= 1.5e-7 -- four orders of magnitude below the bf16
// rounding applied to the result.  The 1/2, the 1/sqrt(2) and log2(e) are folded
// into the constants; exp(-z^2) = 2^(-x^2 log2(e) / 2) goes straight to the
// hardware exp2, whose flush of tiny results only drops terms far below the
// bf16 resolution of x.
__device__ __forceinline__ float gelu_bf16_path(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(ax, 0.3275911f * 0.70710678118654752f, 1.0f));
  float poly = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  poly = fmaf(t, poly, 0.5f * 1.421413741f);
  poly = fmaf(t, poly, 0.5f * -0.284496736f);
  poly = fmaf(t, poly, 0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f((x * -0.72134752044448170f) * x);
  const float h = (poly * t) * e;
  return fmaf(-ax, h, fmaxf(x, 0.f));
}

}  // namespace cem
