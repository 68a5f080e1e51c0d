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
  int gelu;            // 1: GELU after the bias
  int residual;        // 1: add the existing output value
  RowMap rows;
  // residual kind only, nullable: per-row statistics of the rounded output, one
  // (mean, sum of squared deviations) pair per 64-column piece, piece p of row m
  // at stats[2 (p M + m)]
  float* stats = nullptr;
};

enum class Act { None, Gelu };

// OCP e4m3 quantization of one row (the format of gfx950's 8-bit matrix-core
// operands): scale = amax / 448, codes = e4m3(clamp(v * (448 / amax), +-448)),
// rounded to nearest even by the hardware conversion; an all-zero row gets scale 1.
__device__ __forceinline__ void fp8_row_scale(float amax, float& inv, float& scale) {
  const bool zero = !(amax > 0.f);
  const float safe = zero ? 448.0f : amax;
  inv = 448.0f / safe;
  scale = zero ? 1.0f : safe / 448.0f;
}
// eight values -> eight codes (little-endian in a uint2)
__device__ __forceinline__ uint2 fp8x8(const float v[8], float inv) {
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = fminf(fmaxf(v[i] * inv, -448.0f), 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// GELU(x) = x * Phi(x) with Phi from the exact erf (libm erff): fp32 models.
__device__ __forceinline__ float gelu_exact(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// GELU(x) = x * Phi(x) for bf16 models: Phi(x) ~= sigmoid(x q(x^2)), q a quadratic
// fitted (minimax on the absolute error over |x| <= 10) to the exact erf form.
// The result is within 2.6e-5 of exact GELU for every x: about 1/150 of the bf16
// rounding bound (half the spacing) at 1 and 1/19 of it at GELU's minimum
// (-0.17); the bf16 store rounds it right after.  x^2 is capped at 30, where q is still positive and the
// sigmoid is saturated to below 1e-7.  -log2(e) is folded into q, so the
// sigmoid is one hardware exp2 and one reciprocal; large negative x gives
// exp2 -> inf, rcp -> 0, and the exact -0.
__device__ __forceinline__ float gelu_bf16_path(float x) {
  const float u = fminf(x * x, 30.0f);
  const float s = fmaf(fmaf(u, 0.001014263f, -0.10677572f), u, -2.3011212f);
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * s));
}

}  // namespace cem
