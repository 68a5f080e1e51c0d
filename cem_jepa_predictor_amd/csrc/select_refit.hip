// Top-K elite selection and Gaussian refit.
//
// Page "Real-Time Inference for JEPA World Model Architectures with Ray",
// section 01: after scoring, the search keeps the best 80 of the 800
// candidates and re-centres the Gaussian on them.  Selection key: the 64-bit
// word (orderable(energy) << 32) | index, so equal energies rank by index and
// the elite list is unique; NaN ranks as +inf and -0 as +0.  Refit: mean and
// population std of the elites' clamped samples per (step, action dim),
// accumulated in float64 in elite order, rounded to float32.
//
// One 1024-thread workgroup: a bitonic sort of the padded key array in LDS
// (n <= 16384 keys = 128 KB), then the first k keys give the elites.  The refit
// spreads the gather of the elites' samples over the whole workgroup: for
// h * a <= 1024, P = 1024 / (h * a) threads per (step, action dim) each sum the
// elites P apart, and the P partial sums are added in a fixed order (float64
// throughout), so the result is deterministic.  The whole step is a few
// microseconds: it is launch-latency bound.
#include "kernels.hpp"

namespace cem {
namespace {

constexpr int kRefitThreads = 1024;   // the workgroup; also the partial-sum slots
// LDS beyond the keys: kRefitThreads partial sums and up to kRefitThreads means
constexpr int kRefitLds = 2 * kRefitThreads * (int)sizeof(double);

__device__ __forceinline__ uint64_t select_key(float e, int i) {
  uint32_t u = __float_as_uint(e);
  if (e != e) u = 0x7f800000u;          // NaN ranks as +inf
  if (u == 0x80000000u) u = 0u;          // -0 ranks as +0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)i;
}

__global__ __launch_bounds__(kRefitThreads) void select_refit_kernel(const float* __restrict__ E,
                                                            const float* __restrict__ X, int n,
                                                            int npad, int k, int ha,
                                                            int* __restrict__ idx,
                                                            float* __restrict__ mu,
                                                            float* __restrict__ sigma) {
  extern __shared__ uint64_t keys[];
  const int tid = threadIdx.x;
  {  // problem b of a batch: one workgroup each
    const int b = blockIdx.x;
    E += (long long)b * n;
    if (X) X += (long long)b * n * ha;
    idx += (long long)b * k;
    if (mu) { mu += (long long)b * ha; sigma += (long long)b * ha; }
  }
  for (int i = tid; i < npad; i += blockDim.x) keys[i] = i < n ? select_key(E[i], i) : ~0ull;
  __syncthreads();
  for (int size = 2; size <= npad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (npad >> 1); i += blockDim.x) {
        const int lo = (i / stride) * 2 * stride + (i % stride), hi = lo + stride;
        const bool ascending = (lo & size) == 0;
        const uint64_t a = keys[lo], b = keys[hi];
        if ((a > b) == ascending) { keys[lo] = b; keys[hi] = a; }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += blockDim.x) idx[i] = (int)(uint32_t)keys[i];
  if (mu && ha <= kRefitThreads) {
    // LDS after the keys: P x ha partial sums, then ha means (float64)
    double* part = reinterpret_cast<double*>(keys + npad);
    double* mean = part + kRefitThreads;
    const int P = kRefitThreads / ha, j = tid % ha, prt = tid / ha;
    auto xel = [&](int i) { return (double)X[(long long)(uint32_t)keys[i] * ha + j]; };
    if (prt < P) {
      double s = 0.0;
      for (int i = prt; i < k; i += P) s += xel(i);
      part[prt * ha + j] = s;
    }
    __syncthreads();
    if (tid < ha) {
      double s = 0.0;
      for (int q = 0; q < P; ++q) s += part[q * ha + tid];
      mean[tid] = s / (double)k;
    }
    __syncthreads();
    if (prt < P) {
      const double m = mean[j];
      double v = 0.0;
      for (int i = prt; i < k; i += P) {
        const double dlt = xel(i) - m;
        v += dlt * dlt;
      }
      part[prt * ha + j] = v;
    }
    __syncthreads();
    if (tid < ha) {
      double v = 0.0;
      for (int q = 0; q < P; ++q) v += part[q * ha + tid];
      mu[tid] = (float)mean[tid];
      sigma[tid] = (float)sqrt(v / (double)k);
    }
  } else if (mu) {
    for (int j = tid; j < ha; j += blockDim.x) {
      double s = 0.0;
      for (int i = 0; i < k; ++i) s += (double)X[(long long)(uint32_t)keys[i] * ha + j];
      const double mean = s / (double)k;
      double v = 0.0;
      for (int i = 0; i < k; ++i) {
        const double dlt = (double)X[(long long)(uint32_t)keys[i] * ha + j] - mean;
        v += dlt * dlt;
      }
      mu[j] = (float)mean;
      sigma[j] = (float)sqrt(v / (double)k);
    }
  }
}

// Warm start of the next control step (page section 06, "B. Warm-started CEM"):
// receding-horizon control executes only mu_R[0]; steps 1 .. h-1 of the plan seed
// the next step's Gaussian, one step earlier, and the last step starts fresh.
// One workgroup: every element is read before any is written, so the output may
// alias the input.
__global__ __launch_bounds__(1024) void warm_start_kernel(const float* mu_prev,
                                                          const float* sigma_prev, int ha, int a,
                                                          float mu_fill, float sigma_fill,
                                                          float sigma_floor, float* mu_next,
                                                          float* sigma_next) {
  const int i = threadIdx.x;
  float m = mu_fill, s = sigma_fill;
  if (i + a < ha) {
    m = mu_prev[i + a];
    s = fmaxf(sigma_prev[i + a], sigma_floor);   // NaN width -> sigma_floor
  }
  __syncthreads();
  if (i < ha) {
    mu_next[i] = m;
    sigma_next[i] = s;
  }
}

}  // namespace

hipError_t launch_warm_start(const float* mu_prev, const float* sigma_prev, int h, int a,
                             float mu_fill, float sigma_fill, float sigma_floor, float* mu_next,
                             float* sigma_next, hipStream_t stream) {
  const int ha = h * a;
  if (ha <= 0 || ha > 1024) return hipErrorInvalidValue;
  warm_start_kernel<<<1, 1024, 0, stream>>>(mu_prev, sigma_prev, ha, a, mu_fill, sigma_fill,
                                            sigma_floor, mu_next, sigma_next);
  return hipGetLastError();
}

hipError_t select_init() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&select_refit_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             kMaxSelect * (int)sizeof(uint64_t) + kRefitLds);
}

hipError_t launch_select_refit(const float* E, const float* X, int n, int k, int ha, int* idx,
                               float* mu, float* sigma, hipStream_t stream, int batch) {
  if (n <= 0 || k <= 0 || batch <= 0) return hipSuccess;
  int npad = 2;
  while (npad < n) npad <<= 1;
  const size_t lds = npad * sizeof(uint64_t) + (mu ? kRefitLds : 0);
  select_refit_kernel<<<batch, kRefitThreads, lds, stream>>>(E, X, n, npad, k, ha, idx, mu, sigma);
  return hipGetLastError();
}

}  // namespace cem
