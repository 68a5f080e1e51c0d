// L1 energy of each predicted embedding against the goal embedding.
//
// Page "Real-Time Inference for JEPA World Model Architectures with Ray",
// section 01: each rollout result is scored against the goal embedding and
// the candidates closest to it are kept.  Energy = mean over the P x E
// elements of |z_pred - z_goal|, accumulated in fp32.
//
// One 256-thread workgroup per candidate; each lane strides over 16-byte
// vectors of z_pred (the goal, P*E*4 bytes, stays in L2 across candidates);
// the reduction order is fixed (per-lane sums, xor-butterfly within each
// wave64, then the 4 wave sums in order), so results are deterministic.
// HBM-bound: reads N*P*E model-dtype values once.
#include "kernels.hpp"

namespace cem {
namespace {

template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  __device__ static __forceinline__ float absdiff_sum(const bf16* z, const float* g) {
    const uint4 u = *reinterpret_cast<const uint4*>(z);
    const float4 g0 = *reinterpret_cast<const float4*>(g);
    const float4 g1 = *reinterpret_cast<const float4*>(g + 4);
    float s = fabsf(__uint_as_float(u.x << 16) - g0.x) + fabsf(__uint_as_float(u.x & 0xffff0000u) - g0.y);
    s += fabsf(__uint_as_float(u.y << 16) - g0.z) + fabsf(__uint_as_float(u.y & 0xffff0000u) - g0.w);
    s += fabsf(__uint_as_float(u.z << 16) - g1.x) + fabsf(__uint_as_float(u.z & 0xffff0000u) - g1.y);
    s += fabsf(__uint_as_float(u.w << 16) - g1.z) + fabsf(__uint_as_float(u.w & 0xffff0000u) - g1.w);
    return s;
  }
};
template <> struct Vec8<float> {
  __device__ static __forceinline__ float absdiff_sum(const float* z, const float* g) {
    const float4 a0 = *reinterpret_cast<const float4*>(z);
    const float4 a1 = *reinterpret_cast<const float4*>(z + 4);
    const float4 g0 = *reinterpret_cast<const float4*>(g);
    const float4 g1 = *reinterpret_cast<const float4*>(g + 4);
    float s = fabsf(a0.x - g0.x) + fabsf(a0.y - g0.y);
    s += fabsf(a0.z - g0.z) + fabsf(a0.w - g0.w);
    s += fabsf(a1.x - g1.x) + fabsf(a1.y - g1.y);
    s += fabsf(a1.z - g1.z) + fabsf(a1.w - g1.w);
    return s;
  }
};

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void energy_kernel(const T* __restrict__ zp,
                                                     const float* __restrict__ g, long long pe,
                                                     float* __restrict__ E, int n_per) {
  __shared__ float part[4];
  const T* z = zp + (long long)blockIdx.x * pe;
  g += (long long)(blockIdx.x / n_per) * pe;   // this candidate's problem
  float acc = 0.f;
  if (VEC) {
    for (long long j = (long long)threadIdx.x * 8; j < pe; j += 256 * 8)
      acc += Vec8<T>::absdiff_sum(z + j, g + j);
  } else {
    for (long long j = threadIdx.x; j < pe; j += 256) acc += fabsf(Elem<T>::load(z + j) - g[j]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float s = ((part[0] + part[1]) + part[2]) + part[3];
    E[blockIdx.x] = (float)((double)s / (double)pe);
  }
}

}  // namespace

template <typename T>
hipError_t launch_energy(const T* zp, const float* g, int n, long long pe, float* E, int n_per,
                         hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (n_per <= 0) return hipErrorInvalidValue;
  const bool vec = (pe % 8 == 0) && ((uintptr_t)zp % 16 == 0) && ((uintptr_t)g % 16 == 0);
  if (vec)
    energy_kernel<T, true><<<n, 256, 0, stream>>>(zp, g, pe, E, n_per);
  else
    energy_kernel<T, false><<<n, 256, 0, stream>>>(zp, g, pe, E, n_per);
  return hipGetLastError();
}

template hipError_t launch_energy<float>(const float*, const float*, int, long long, float*, int,
                                         hipStream_t);
template hipError_t launch_energy<bf16>(const bf16*, const float*, int, long long, float*, int,
                                        hipStream_t);

}  // namespace cem
