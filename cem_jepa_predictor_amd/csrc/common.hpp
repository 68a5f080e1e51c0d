// Shared device/host definitions of the gfx950 CEM library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cem {

using bf16 = uint16_t;   // storage type: upper 16 bits of an IEEE binary32

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16 v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest, ties to even (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<bf16>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16>(u >> 16);
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

__device__ __forceinline__ float gelu_exact(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

}  // namespace cem
