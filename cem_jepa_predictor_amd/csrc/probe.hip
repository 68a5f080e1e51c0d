// Sustained matrix-core ceiling of the part the library runs on.
//
// The dense projections are compared against the published bf16 peak, but
// the clock under full MFMA load depends on power: with operands whose bits
// change every instruction (as real activations and weights do) the part
// settles well below its nominal clock.  This kernel measures that ceiling:
// every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on register-resident
// operands (four A and four B fragments cycled, eight independent
// accumulators), no memory traffic inside the timed loop.  One workgroup of
// four waves per CU.  Each workgroup also records its shader-clock cycles and
// constant-rate (100 MHz) wall ticks, which give the clock it ran at.
#include "cem_probe.h"
#include "kernels.hpp"

namespace cem {
namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* sink, unsigned long long* ticks,
                                                                   int iters, int random_operands) {
  bf16x8_t a[4], b[4];
  uint32_t h = threadIdx.x * 2654435761u + blockIdx.x * 97u + 12345u;
  auto next = [&]() {   // xorshift32
    h ^= h << 13; h ^= h >> 17; h ^= h << 5;
    return h;
  };
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float fa = random_operands ? (float)(next() & 0xffff) / 32768.0f - 1.0f : 0.5f;
      const float fb = random_operands ? ((float)(next() & 0xffff) / 32768.0f - 1.0f) * 0.02f : 0.01f;
      a[k][i] = (__bf16)fa;
      b[k][i] = (__bf16)fb;
    }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc[j & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j >> 2) & 3], acc[j & 7], 0, 0, 0);
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = c1 - c0;
    ticks[2 * blockIdx.x + 1] = w1 - w0;
  }
}

}  // namespace

hipError_t mfma_ceiling(int random_operands, int launches, double* tflops, double* mhz) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int blocks = cus, iters = 20000;
  float* sink = nullptr;
  unsigned long long* ticks = nullptr;
  hipStream_t st = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  auto cleanup = [&]() {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (st) (void)hipStreamDestroy(st);
    if (sink) (void)hipFree(sink);
    if (ticks) (void)hipFree(ticks);
  };
#define PROBE_TRY(x) do { e = (x); if (e != hipSuccess) { cleanup(); return e; } } while (0)
  PROBE_TRY(hipMalloc(&sink, (size_t)blocks * kProbeThreads * sizeof(float)));
  PROBE_TRY(hipMalloc(&ticks, (size_t)blocks * 2 * sizeof(unsigned long long)));
  PROBE_TRY(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
  PROBE_TRY(hipEventCreate(&e0));
  PROBE_TRY(hipEventCreate(&e1));
  // the first half of the launches brings the clock to its steady state; the
  // second half is timed
  const int warm = launches / 2, timed = launches - warm;
  for (int i = 0; i < warm; ++i)
    mfma_probe_kernel<<<blocks, kProbeThreads, 0, st>>>(sink, ticks, iters, random_operands);
  PROBE_TRY(hipGetLastError());
  PROBE_TRY(hipEventRecord(e0, st));
  for (int i = 0; i < timed; ++i)
    mfma_probe_kernel<<<blocks, kProbeThreads, 0, st>>>(sink, ticks, iters, random_operands);
  PROBE_TRY(hipGetLastError());
  PROBE_TRY(hipEventRecord(e1, st));
  PROBE_TRY(hipEventSynchronize(e1));
  float ms = 0.f;
  PROBE_TRY(hipEventElapsedTime(&ms, e0, e1));
  unsigned long long t[2] = {0, 0};
  PROBE_TRY(hipMemcpy(t, ticks, sizeof(t), hipMemcpyDeviceToHost));
#undef PROBE_TRY
  cleanup();
  const double flop = (double)timed * blocks * (kProbeThreads / 64) * (double)iters * 16 * (2.0 * 32 * 32 * 16);
  *tflops = flop / (ms * 1e-3) / 1e12;
  *mhz = t[1] ? (double)t[0] / ((double)t[1] / 100.0) : 0.0;
  return hipSuccess;
}

}  // namespace cem

extern "C" cem_status cem_mfma_ceiling(int32_t random_operands, int32_t launches, double* tflops,
                                       double* mhz) {
  if (!tflops || !mhz) return CEM_E_ARG;
  if (random_operands != 0 && random_operands != 1) return CEM_E_ARG;
  if (launches < 2 || launches > 10000) return CEM_E_ARG;
  return cem::mfma_ceiling(random_operands, launches, tflops, mhz) == hipSuccess ? CEM_OK : CEM_E_HIP;
}
