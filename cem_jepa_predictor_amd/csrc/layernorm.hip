// LayerNorm over rows of the residual stream (fp32 statistics).
//
// The predictor is a pre-LayerNorm transformer: each block normalises its
// input before attention and before the MLP, and the final patch rows are
// normalised before the out-projection (the V-JEPA2-AC predictor of page "Real-
// Time Inference for JEPA World Model Architectures with Ray", section 01,
// with the sizes of that predictor).  Mean and biased variance in fp32, exact
// two-pass in registers; y = (x - mean) * rsqrt(var + eps) * g + b.
//
// One 64-lane wavefront per row; each lane owns 2*NCH elements as NCH pairs
// (d = 128 * NCH).  HBM-bound: reads d and writes d elements per row.
#include "kernels.hpp"

namespace cem {
namespace {

template <typename T> struct Pair;
template <> struct Pair<float> {
  using V = float2;
  __device__ static __forceinline__ void unpack(V v, float& a, float& b) { a = v.x; b = v.y; }
  __device__ static __forceinline__ V pack(float a, float b) { return make_float2(a, b); }
};
template <> struct Pair<bf16> {
  using V = uint32_t;
  __device__ static __forceinline__ void unpack(V v, float& a, float& b) {
    a = __uint_as_float(v << 16);
    b = __uint_as_float(v & 0xffff0000u);
  }
  __device__ static __forceinline__ V pack(float a, float b) { return pack_bf16x2(a, b); }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int NCH, typename T>
__global__ __launch_bounds__(256) void layernorm_kernel(const T* __restrict__ x, int rows,
                                                        RowMap in_rows,
                                                        const float* __restrict__ g,
                                                        const float* __restrict__ b, float eps,
                                                        T* __restrict__ y) {
  using P = Pair<T>;
  constexpr int d = 128 * NCH;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const typename P::V* src = reinterpret_cast<const typename P::V*>(x + in_rows(r) * (long long)d);
  float v[2 * NCH];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    P::unpack(src[c * 64 + lane], v[2 * c], v[2 * c + 1]);
    s += v[2 * c] + v[2 * c + 1];
  }
  const float mean = wave_sum(s) * (1.0f / d);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 2 * NCH; ++i) {
    const float t = v[i] - mean;
    q += t * t;
  }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / d) + eps);
  typename P::V* dst = reinterpret_cast<typename P::V*>(y + (long long)r * d);
  const float2* g2 = reinterpret_cast<const float2*>(g);
  const float2* b2 = reinterpret_cast<const float2*>(b);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const float2 gg = g2[c * 64 + lane], bb = b2[c * 64 + lane];
    dst[c * 64 + lane] = P::pack((v[2 * c] - mean) * rstd * gg.x + bb.x,
                                 (v[2 * c + 1] - mean) * rstd * gg.y + bb.y);
  }
}

template <int NCH, typename T>
hipError_t run(const T* x, int rows, RowMap in_rows, const float* g, const float* b, float eps,
               T* y, hipStream_t stream) {
  layernorm_kernel<NCH, T><<<(rows + 3) / 4, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y);
  return hipGetLastError();
}

}  // namespace

bool layernorm_supports(int d) {
  switch (d) {
    case 128: case 256: case 384: case 512: case 768: case 1024: case 1536: case 2048:
    case 4096: return true;
    default: return false;
  }
}

template <typename T>
hipError_t launch_layernorm(const T* x, int rows, int d, RowMap in_rows, const float* g,
                            const float* b, float eps, T* y, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  switch (d) {
    case 128: return run<1>(x, rows, in_rows, g, b, eps, y, stream);
    case 256: return run<2>(x, rows, in_rows, g, b, eps, y, stream);
    case 384: return run<3>(x, rows, in_rows, g, b, eps, y, stream);
    case 512: return run<4>(x, rows, in_rows, g, b, eps, y, stream);
    case 768: return run<6>(x, rows, in_rows, g, b, eps, y, stream);
    case 1024: return run<8>(x, rows, in_rows, g, b, eps, y, stream);
    case 1536: return run<12>(x, rows, in_rows, g, b, eps, y, stream);
    case 2048: return run<16>(x, rows, in_rows, g, b, eps, y, stream);
    case 4096: return run<32>(x, rows, in_rows, g, b, eps, y, stream);
    default: return hipErrorInvalidValue;
  }
}

template hipError_t launch_layernorm<float>(const float*, int, int, RowMap, const float*,
                                            const float*, float, float*, hipStream_t);
template hipError_t launch_layernorm<bf16>(const bf16*, int, int, RowMap, const float*,
                                           const float*, float, bf16*, hipStream_t);

}  // namespace cem
