// Gaussian candidate sampler: Philox-4x32-10 -> float64 Box-Muller -> clamp.
//
// Page "Real-Time Inference for JEPA World Model Architectures with Ray",
// section 01: every round draws the candidate action sequences from a Gaussian
// centred on the current best guess.  Philox-4x32-10 is the counter-based
// generator of Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11); its multipliers and Weyl key increments are the 4x32 constants
// given there.  Element e of the [n, ha] sample uses counter
// (e >> 2, round, plan_id, 0) under key (seed lo, seed hi); words w0, w1 serve
// e & 3 in {0, 1} and w2, w3 serve {2, 3}; u1 = (w_even + 1) 2^-32,
// u2 = w_odd 2^-32, z_even = sqrt(-2 ln u1) cos(2 pi u2), z_odd = ... sin(...),
// in float64, then rounded to float32.  x = clamp(mu + sigma z) with one
// float32 rounding per operation (this file is built with -ffp-contract=off).
//
// One thread per Philox counter: 4 elements, 10 rounds of 32x32->64 multiplies.
// The sample is tiny (N*H*A floats); the kernel is launch-latency bound.
#include "kernels.hpp"

namespace cem {
namespace {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct Words { uint32_t w[4]; };

__device__ __forceinline__ Words philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += kPhiloxW0; k1 += kPhiloxW1; }
    const uint32_t hi0 = __umulhi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint32_t hi1 = __umulhi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return Words{{c0, c1, c2, c3}};
}

__device__ __forceinline__ void box_muller(uint32_t we, uint32_t wo, float& ze, float& zo) {
  const double u1 = ((double)we + 1.0) * 0x1p-32;
  const double u2 = (double)wo * 0x1p-32;
  const double rho = sqrt(-2.0 * log(u1));
  const double theta = (2.0 * 3.141592653589793) * u2;
  ze = (float)(rho * cos(theta));
  zo = (float)(rho * sin(theta));
}

__global__ __launch_bounds__(256) void sample_kernel(const float* __restrict__ mu,
                                                     const float* __restrict__ sigma, int total,
                                                     int ha, uint32_t k0, uint32_t k1,
                                                     uint32_t round, uint32_t plan_id,
                                                     const uint32_t* __restrict__ dev_params,
                                                     float lo, float hi, float* __restrict__ x,
                                                     uint32_t* __restrict__ raw) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * c >= total) return;
  if (dev_params) {
    k0 = dev_params[0]; k1 = dev_params[1]; plan_id = dev_params[2];
    round += dev_params[3];   // the plan's first round
  }
  // problem b of a batch: its own Gaussian and sample block, plan id + b
  const int b = blockIdx.y;
  plan_id += (uint32_t)b;
  mu += (long long)b * ha;
  sigma += (long long)b * ha;
  x += (long long)b * total;
  if (raw) raw += (long long)b * total;
  const Words w = philox4x32_10((uint32_t)c, round, plan_id, 0u, k0, k1);
  float z[4];
  box_muller(w.w[0], w.w[1], z[0], z[1]);
  box_muller(w.w[2], w.w[3], z[2], z[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * c + j;
    if (e < total) {
      const int col = e % ha;
      const float v = __fadd_rn(mu[col], __fmul_rn(sigma[col], z[j]));
      x[e] = fminf(fmaxf(v, lo), hi);
      if (raw) raw[e] = w.w[j];
    }
  }
}

__global__ void set_params_kernel(uint32_t* p, uint32_t k0, uint32_t k1, uint32_t plan_id,
                                  uint32_t first_round) {
  if (threadIdx.x == 0) { p[0] = k0; p[1] = k1; p[2] = plan_id; p[3] = first_round; }
}

}  // namespace

hipError_t launch_sample(const float* mu, const float* sigma, int n, int ha, uint64_t seed,
                         uint32_t round, uint32_t plan_id, const uint32_t* dev_params, float lo,
                         float hi, float* x, uint32_t* raw, hipStream_t stream, int batch) {
  const int total = n * ha;
  if (total <= 0 || batch <= 0) return hipSuccess;
  const int counters = (total + 3) / 4;
  const dim3 blocks((unsigned)((counters + 255) / 256), (unsigned)batch);
  sample_kernel<<<blocks, 256, 0, stream>>>(mu, sigma, total, ha, (uint32_t)seed,
                                            (uint32_t)(seed >> 32), round, plan_id, dev_params,
                                            lo, hi, x, raw);
  return hipGetLastError();
}

hipError_t launch_set_params(uint32_t* dev_params, uint64_t seed, uint32_t plan_id,
                             uint32_t first_round, hipStream_t stream) {
  set_params_kernel<<<1, 64, 0, stream>>>(dev_params, (uint32_t)seed, (uint32_t)(seed >> 32),
                                          plan_id, first_round);
  return hipGetLastError();
}

}  // namespace cem
