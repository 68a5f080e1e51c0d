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
// (d = 128 * NCH), or for bf16 rows with d % 512 == 0, runs of 8 elements moved
// with 16-byte accesses.  HBM-bound: reads d and writes d elements per row.
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

// Sum and max over the 64 lanes, the same value in every lane, without LDS: lanes
// combine in pairs through DPP quad permutations ([1,0,3,2], [2,3,0,1]) and the
// half-row and row mirrors (within 16 lanes), then across 16-lane rows through
// v_permlane16_swap and across the two halves through v_permlane32_swap.  Each step
// combines two lanes' values, which both lanes get bit for bit (the operation is
// commutative).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_f<0xb1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_f<0x4e>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_f<0x141>(v));   // row_half_mirror
  v = op(v, dpp_f<0x140>(v));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
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

// bf16 rows with d = 512 * NC: each lane owns NC runs of 8 consecutive elements
// (16-byte loads and stores, one 1 KB wave access per run).
template <int NC>
__global__ __launch_bounds__(256) void layernorm_bf16x8_kernel(const bf16* __restrict__ x, int rows,
                                                               RowMap in_rows,
                                                               const float* __restrict__ g,
                                                               const float* __restrict__ b, float eps,
                                                               bf16* __restrict__ y) {
  constexpr int d = 512 * NC;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + in_rows(r) * (long long)d);
  float v[8 * NC];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint4 u = src[c * 64 + lane];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * c + 2 * k] = __uint_as_float(w[k] << 16);
      v[8 * c + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      s += v[8 * c + 2 * k] + v[8 * c + 2 * k + 1];
    }
  }
  const float mean = wave_sum(s) * (1.0f / d);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 8 * NC; ++i) {
    const float t = v[i] - mean;
    q += t * t;
  }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / d) + eps);
  uint4* dst = reinterpret_cast<uint4*>(y + (long long)r * d);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float4 g0 = g4[(c * 64 + lane) * 2], g1 = g4[(c * 64 + lane) * 2 + 1];
    const float4 b0 = b4[(c * 64 + lane) * 2], b1 = b4[(c * 64 + lane) * 2 + 1];
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = pack_bf16x2((v[8 * c + 2 * k] - mean) * rstd * gg[2 * k] + bb[2 * k],
                         (v[8 * c + 2 * k + 1] - mean) * rstd * gg[2 * k + 1] + bb[2 * k + 1]);
    dst[c * 64 + lane] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

// LayerNorm of bf16 rows (d = 512 * NC, one wave per row, 8 consecutive values per
// lane run) with OCP e4m3 output, scaled per row by 448 / amax of the normalised row.
template <int NC>
__global__ __launch_bounds__(256) void layernorm_fp8_kernel(const bf16* __restrict__ x, int rows,
                                                            RowMap in_rows,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ b, float eps,
                                                            uint8_t* __restrict__ y8,
                                                            float* __restrict__ row_scale) {
  constexpr int d = 512 * NC;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + in_rows(r) * (long long)d);
  float v[8 * NC];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint4 u = src[c * 64 + lane];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * c + 2 * k] = __uint_as_float(w[k] << 16);
      v[8 * c + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      s += v[8 * c + 2 * k] + v[8 * c + 2 * k + 1];
    }
  }
  const float mean = wave_sum(s) * (1.0f / d);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 8 * NC; ++i) {
    const float t = v[i] - mean;
    q += t * t;
  }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / d) + eps);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float4 g0 = g4[(c * 64 + lane) * 2], g1 = g4[(c * 64 + lane) * 2 + 1];
    const float4 b0 = b4[(c * 64 + lane) * 2], b1 = b4[(c * 64 + lane) * 2 + 1];
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[8 * c + k] = (v[8 * c + k] - mean) * rstd * gg[k] + bb[k];
      amax = fmaxf(amax, fabsf(v[8 * c + k]));
    }
  }
  float inv, scale;
  fp8_row_scale(wave_max(amax), inv, scale);
  uint2* dst = reinterpret_cast<uint2*>(y8 + (long long)r * d);
#pragma unroll
  for (int c = 0; c < NC; ++c) dst[c * 64 + lane] = fp8x8(v + 8 * c, inv);
  if (lane == 0) row_scale[r] = scale;
}

// Per-row e4m3 quantization of fp32 rows [rows, cols], cols % 8 == 0: one wave per row.
__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(const float* __restrict__ x, int rows,
                                                                int cols, uint8_t* __restrict__ y8,
                                                                float* __restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = x + (long long)r * cols;
  float amax = 0.f;
  for (int c = lane * 8; c < cols; c += 512)
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(xr[c + k]));
  float inv, scale;
  fp8_row_scale(wave_max(amax), inv, scale);
  for (int c = lane * 8; c < cols; c += 512) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = xr[c + k];
    *reinterpret_cast<uint2*>(y8 + (long long)r * cols + c) = fp8x8(v, inv);
  }
  if (lane == 0) row_scale[r] = scale;
}

// Row statistics only (a LayerNorm folded into the GEMM that consumes its rows):
// mean and rstd of bf16 rows with the arithmetic of the kernels above.  VEC = 8:
// d = 512 * N, 16-byte runs; VEC = 2: d = 128 * N, bf16 pairs.  Reads d elements
// and writes 8 bytes per row.
template <int VEC, int N>
__global__ __launch_bounds__(256) void row_stats_kernel(const bf16* __restrict__ x, int rows,
                                                        float eps, float* __restrict__ mean_out,
                                                        float* __restrict__ rstd_out) {
  constexpr int d = 64 * VEC * N;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float v[VEC * N];
  float s = 0.f;
  if constexpr (VEC == 8) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (long long)r * d);
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const uint4 u = src[c * 64 + lane];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * c + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * c + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        s += v[8 * c + 2 * k] + v[8 * c + 2 * k + 1];
      }
    }
  } else {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(x + (long long)r * d);
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const uint32_t u = src[c * 64 + lane];
      v[2 * c] = __uint_as_float(u << 16);
      v[2 * c + 1] = __uint_as_float(u & 0xffff0000u);
      s += v[2 * c] + v[2 * c + 1];
    }
  }
  const float mean = wave_sum(s) * (1.0f / d);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VEC * N; ++i) {
    const float t = v[i] - mean;
    q += t * t;
  }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / d) + eps);
  if (lane == 0) {
    mean_out[r] = mean;
    rstd_out[r] = rstd;
  }
}

// Row statistics from partial statistics of 64-column pieces, written by the
// residual GEMM that produced the rows: piece p of row r holds the mean and the
// sum of squared deviations of its 64 values at parts[2 (p rows + r)].  Exact
// decomposition of the same two quantities over the whole row: the mean is the
// average of the piece means, and the sum of squared deviations is the sum over
// pieces of (piece sum + 64 (piece mean - mean)^2).  One thread per row, all P
// pieces loaded at once (8 bytes per piece and row, coalesced across the rows of
// a piece); P = 0: the piece count comes at run time and the pieces are read twice.
template <int P>
__global__ __launch_bounds__(256) void row_stats_combine_kernel(const float2* __restrict__ parts,
                                                                int pieces, int rows, float eps,
                                                                float* __restrict__ mean_out,
                                                                float* __restrict__ rstd_out) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int np = P > 0 ? P : pieces;
  float mean, q = 0.f;
  if constexpr (P > 0) {
    float2 v[P];
#pragma unroll
    for (int p = 0; p < P; ++p) v[p] = parts[(long long)p * rows + r];
    float sm = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) sm += v[p].x;
    mean = sm / (float)P;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float dm = v[p].x - mean;
      q += fmaf(64.0f * dm, dm, v[p].y);
    }
  } else {
    float sm = 0.f;
    for (int p = 0; p < np; ++p) sm += parts[(long long)p * rows + r].x;
    mean = sm / (float)np;
    for (int p = 0; p < np; ++p) {
      const float2 v = parts[(long long)p * rows + r];
      const float dm = v.x - mean;
      q += fmaf(64.0f * dm, dm, v.y);
    }
  }
  mean_out[r] = mean;
  rstd_out[r] = rsqrtf(q / (64.0f * (float)np) + eps);
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
  if constexpr (sizeof(T) == 2) {
    // 16-byte path: x rows (and so g, b, y) are 16-byte aligned when d % 512 == 0
    const int grid = (rows + 3) / 4;
    if (d == 1024) {
      layernorm_bf16x8_kernel<2><<<grid, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y);
      return hipGetLastError();
    }
    if (d == 512) {
      layernorm_bf16x8_kernel<1><<<grid, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y);
      return hipGetLastError();
    }
    if (d == 2048) {
      layernorm_bf16x8_kernel<4><<<grid, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y);
      return hipGetLastError();
    }
  }
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

hipError_t launch_layernorm_fp8(const bf16* x, int rows, int d, RowMap in_rows, const float* g,
                                const float* b, float eps, uint8_t* y8, float* row_scale,
                                hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int grid = (rows + 3) / 4;
  switch (d) {
    case 512: layernorm_fp8_kernel<1><<<grid, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y8, row_scale); break;
    case 1024: layernorm_fp8_kernel<2><<<grid, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y8, row_scale); break;
    case 1536: layernorm_fp8_kernel<3><<<grid, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y8, row_scale); break;
    case 2048: layernorm_fp8_kernel<4><<<grid, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y8, row_scale); break;
    case 4096: layernorm_fp8_kernel<8><<<grid, 256, 0, stream>>>(x, rows, in_rows, g, b, eps, y8, row_scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_row_stats(const bf16* x, int rows, int d, float eps, float* mean, float* rstd,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int grid = (rows + 3) / 4;
#define CEM_STATS(V, N) row_stats_kernel<V, N><<<grid, 256, 0, stream>>>(x, rows, eps, mean, rstd); break
  switch (d) {
    case 128: CEM_STATS(2, 1);
    case 256: CEM_STATS(2, 2);
    case 384: CEM_STATS(2, 3);
    case 512: CEM_STATS(8, 1);
    case 768: CEM_STATS(2, 6);
    case 1024: CEM_STATS(8, 2);
    case 1536: CEM_STATS(8, 3);
    case 2048: CEM_STATS(8, 4);
    case 4096: CEM_STATS(8, 8);
    default: return hipErrorInvalidValue;
  }
#undef CEM_STATS
  return hipGetLastError();
}

hipError_t launch_row_stats_combine(const float* parts, int rows, int d, float eps, float* mean,
                                    float* rstd, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (d <= 0 || d % 64 != 0 || !parts) return hipErrorInvalidValue;
  const float2* pp = reinterpret_cast<const float2*>(parts);
  const int grid = (rows + 255) / 256;
  switch (d / 64) {
    case 8: row_stats_combine_kernel<8><<<grid, 256, 0, stream>>>(pp, 8, rows, eps, mean, rstd); break;
    case 16: row_stats_combine_kernel<16><<<grid, 256, 0, stream>>>(pp, 16, rows, eps, mean, rstd); break;
    case 32: row_stats_combine_kernel<32><<<grid, 256, 0, stream>>>(pp, 32, rows, eps, mean, rstd); break;
    default: row_stats_combine_kernel<0><<<grid, 256, 0, stream>>>(pp, d / 64, rows, eps, mean, rstd);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rows_fp8(const float* x, int rows, int cols, uint8_t* y8,
                                    float* row_scale, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (cols <= 0 || cols % 8 != 0) return hipErrorInvalidValue;
  quantize_rows_fp8_kernel<<<(rows + 3) / 4, 256, 0, stream>>>(x, rows, cols, y8, row_scale);
  return hipGetLastError();
}

template hipError_t launch_layernorm<float>(const float*, int, int, RowMap, const float*,
                                            const float*, float, float*, hipStream_t);
template hipError_t launch_layernorm<bf16>(const bf16*, int, int, RowMap, const float*,
                                           const float*, float, bf16*, hipStream_t);

}  // namespace cem
