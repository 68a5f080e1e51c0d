// L1 energy of each predicted embedding against the goal embedding.
//
// Page "Real-Time Inference for JEPA World Model Architectures with Ray",
// section 01: each rollout result is scored against the goal embedding and
// the candidates closest to it are kept.  Energy = mean over the P x E
// elements of |z_pred - z_goal|, accumulated in fp32.
//
// One 512-thread workgroup per four candidates of one problem (one per
// candidate when the count does not split into fours): each lane strides over
// 16-byte vectors of z_pred and loads the matching goal vector once for all of
// the workgroup's candidates, so the goal (fp32, twice the bytes of a bf16
// prediction, served from L2) costs a quarter of the load traffic it would
// with one candidate per workgroup.  Each candidate's sum runs in a fixed
// order that does not depend on how many candidates share the workgroup
// (per-lane sums, xor-butterfly within each wave64, then the 8 wave sums in
// order), so results are deterministic and independent of the batch.
// HBM-bound: reads N*P*E model-dtype values once.
#include "kernels.hpp"

namespace cem {
namespace {

// Sum of |z - g| over 8 consecutive elements, in a fixed order.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  __device__ static __forceinline__ float absdiff_sum(const bf16* z, const float4& g0, const float4& g1) {
    const uint4 u = *reinterpret_cast<const uint4*>(z);
    float s = fabsf(__uint_as_float(u.x << 16) - g0.x) + fabsf(__uint_as_float(u.x & 0xffff0000u) - g0.y);
    s += fabsf(__uint_as_float(u.y << 16) - g0.z) + fabsf(__uint_as_float(u.y & 0xffff0000u) - g0.w);
    s += fabsf(__uint_as_float(u.z << 16) - g1.x) + fabsf(__uint_as_float(u.z & 0xffff0000u) - g1.y);
    s += fabsf(__uint_as_float(u.w << 16) - g1.z) + fabsf(__uint_as_float(u.w & 0xffff0000u) - g1.w);
    return s;
  }
};
template <> struct Vec8<float> {
  __device__ static __forceinline__ float absdiff_sum(const float* z, const float4& g0, const float4& g1) {
    const float4 a0 = *reinterpret_cast<const float4*>(z);
    const float4 a1 = *reinterpret_cast<const float4*>(z + 4);
    float s = fabsf(a0.x - g0.x) + fabsf(a0.y - g0.y);
    s += fabsf(a0.z - g0.z) + fabsf(a0.w - g0.w);
    s += fabsf(a1.x - g1.x) + fabsf(a1.y - g1.y);
    s += fabsf(a1.z - g1.z) + fabsf(a1.w - g1.w);
    return s;
  }
};

constexpr int kEnergyThreads = 512, kEnergyWaves = kEnergyThreads / 64;

// C candidates c0 .. c0 + C - 1 (c0 = C * workgroup) of one problem.
template <typename T, bool VEC, int C>
__global__ __launch_bounds__(kEnergyThreads) void energy_kernel(const T* __restrict__ zp,
                                                                const float* __restrict__ g,
                                                                long long pe, float* __restrict__ E,
                                                                int n_per) {
  __shared__ float part[C][kEnergyWaves];
  const int c0 = blockIdx.x * C;
  const T* z = zp + (long long)c0 * pe;
  g += (long long)(c0 / n_per) * pe;   // the candidates' problem
  float acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = 0.f;
  if (VEC) {
    for (long long j = (long long)threadIdx.x * 8; j < pe; j += kEnergyThreads * 8) {
      const float4 g0 = *reinterpret_cast<const float4*>(g + j);
      const float4 g1 = *reinterpret_cast<const float4*>(g + j + 4);
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] += Vec8<T>::absdiff_sum(z + c * pe + j, g0, g1);
    }
  } else {
    for (long long j = threadIdx.x; j < pe; j += kEnergyThreads) {
      const float gj = g[j];
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] += fabsf(Elem<T>::load(z + c * pe + j) - gj);
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc[c] += __shfl_xor(acc[c], o, 64);
    if ((threadIdx.x & 63) == 0) part[c][threadIdx.x >> 6] = acc[c];
  }
  __syncthreads();
  if (threadIdx.x < C) {
    float s = part[threadIdx.x][0];
#pragma unroll
    for (int w = 1; w < kEnergyWaves; ++w) s += part[threadIdx.x][w];
    E[c0 + threadIdx.x] = (float)((double)s / (double)pe);
  }
}

}  // namespace

template <typename T>
hipError_t launch_energy(const T* zp, const float* g, int n, long long pe, float* E, int n_per,
                         hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (n_per <= 0) return hipErrorInvalidValue;
  const bool vec = (pe % 8 == 0) && ((uintptr_t)zp % 16 == 0) && ((uintptr_t)g % 16 == 0);
  if (n % 4 == 0 && n_per % 4 == 0) {   // four candidates per workgroup, all of one problem
    if (vec) energy_kernel<T, true, 4><<<n / 4, kEnergyThreads, 0, stream>>>(zp, g, pe, E, n_per);
    else energy_kernel<T, false, 4><<<n / 4, kEnergyThreads, 0, stream>>>(zp, g, pe, E, n_per);
  } else {
    if (vec) energy_kernel<T, true, 1><<<n, kEnergyThreads, 0, stream>>>(zp, g, pe, E, n_per);
    else energy_kernel<T, false, 1><<<n, kEnergyThreads, 0, stream>>>(zp, g, pe, E, n_per);
  }
  return hipGetLastError();
}

template hipError_t launch_energy<float>(const float*, const float*, int, long long, float*, int,
                                         hipStream_t);
template hipError_t launch_energy<bf16>(const bf16*, const float*, int, long long, float*, int,
                                        hipStream_t);

}  // namespace cem
