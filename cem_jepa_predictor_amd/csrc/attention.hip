// Block-causal multi-head attention of the predictor's current frame block.
//
// Page "Real-Time Inference for JEPA World Model Architectures with Ray",
// section 05: the predictor is frame-causal, so at rollout step t the queries
// of frame block t attend to the keys of blocks 0..t, and the keys/values of
// earlier blocks come from a KV cache instead of being recomputed.  Within a
// block attention is bidirectional.  Softmax scale 1/sqrt(dh), fp32 softmax.
//
// bf16 kernel (dh = 64), one 256-thread workgroup per (candidate, head):
//  * the keys/values of one frame block at a time (B keys, padded to a
//    multiple of 32) are staged in dynamic LDS: K row-major with 16-byte
//    chunks XOR-swizzled by key % 8, V transposed (Vt[dh][key], padded rows) so
//    both MFMA operands are contiguous LDS reads.  74 KB at B = 258, so two
//    workgroups share a CU and one's loads overlap the other's math;
//  * each wave owns 16-row query tiles; per tile and staged block it computes
//    all of S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (lane l holds the scores
//    of query l % 16 in registers), takes the block's exact max, and keeps a
//    running max / sum only across frame blocks (one rescale per block); then
//    O^T += V^T P^T with P taken straight from registers: the MFMA sums over
//    its 32 key slots, and the key each slot stands for is chosen so that the
//    lane's own probabilities and the matching V^T entries line up (any
//    consistent assignment of keys to slots gives the same sum);
//  * HBM traffic per (candidate, head) is one read of Q, K, V and one write of
//    O: the kernel is bandwidth-bound at the V-JEPA2-AC shape.
#include <utility>

#include "kernels.hpp"

namespace cem {
namespace {

constexpr int kDh = 64;
constexpr int kMaxTilesPerWave = 5;  // 16-row query tiles per wave -> B <= 320
constexpr int kMaxKeyTiles = 20;     // 16-key tiles per staged block -> B <= 320

constexpr __host__ __device__ int kpad_of(int B) { return (B + 31) & ~31; }
__host__ __device__ __forceinline__ int vt_ld_of(int B) { return kpad_of(B) + 8; }
__host__ __device__ __forceinline__ int lds_bytes_of(int B) {
  return kpad_of(B) * kDh * 2 + kDh * vt_ld_of(B) * 2;
}

__device__ __forceinline__ float wave_max_q(float v) {
  // lanes l, l^16, l^32, l^48 share query l % 16
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_q(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// One frame block (every query sees exactly the B keys of its own block):
// each query tile computes its full score block in registers, takes the exact
// max, exponentiates once and finishes before the next tile.
// KT = ceil(B / 16): 16-key (and 16-query) tiles per block, fixed per model.
template <int KT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void attn_bf16_single_kernel(AttnArgs p) {
  constexpr int kKT2 = 2 * ((KT + 1) / 2);   // key tiles rounded up to MFMA k = 32 pairs
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int B = p.B, kpad = kpad_of(B), vld = vt_ld_of(B);
  uint8_t* k_lds = lds;
  bf16* vt_lds = reinterpret_cast<bf16*>(lds + kpad * kDh * 2);

  const int n = blockIdx.x / p.heads, h = blockIdx.x % p.heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, ql = lane & 15;
  const float sl2 = p.scale * 1.4426950408889634f;   // softmax in base 2

  const bf16* kvb = static_cast<const bf16*>(p.kv[0]) + (long long)n * B * p.ldkv + h * kDh;
  // Staging: every K and V load of this thread is issued before any LDS store, so
  // the loads' latencies overlap instead of adding up.
  // K: 8 lanes per 128-byte key row (coalesced), 16-byte swizzled LDS stores.
  // V: a wave takes 16 keys x 4 chunks, so each transposed 2-byte store
  // instruction writes 4 Vt rows x 32 contiguous bytes on distinct banks.
  constexpr int kItems = (kpad_of(16 * KT) * 8 + 255) / 256;   // per thread, K and V each
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 kreg[kItems], vreg[kItems];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int item = tid + 256 * it;
    const int kr = item >> 3, ck = item & 7;
    const int vr = (item & 15) + 16 * (item >> 7);
    const int vc = ((item >> 4) & 3) + 4 * ((item >> 6) & 1);
    if (item < kpad * 8) {
      kreg[it] = *reinterpret_cast<const u32x4*>(kvb + (long long)min(kr, B - 1) * p.ldkv + ck * 8);
      vreg[it] = *reinterpret_cast<const u32x4*>(kvb + p.d + (long long)min(vr, B - 1) * p.ldkv + vc * 8);
    }
  }
  // this wave's query fragments (tiles wave, wave + 4, ...), fetched with K and V
  constexpr int kTilesPerWave = (KT + 3) / 4;
  const bf16* qbase = static_cast<const bf16*>(p.q) + (long long)n * B * p.ldq + h * kDh;
  bf16x8_t qall[kTilesPerWave][2];
#pragma unroll
  for (int ti = 0; ti < kTilesPerWave; ++ti) {
    const int qr = min((wave + 4 * ti) * 16 + ql, B - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qall[ti][s] = *reinterpret_cast<const bf16x8_t*>(qbase + (long long)qr * p.ldq + 32 * s + 8 * g);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the first LDS store
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int item = tid + 256 * it;
    if (item < kpad * 8) {
      const int kr = item >> 3, ck = item & 7;
      *reinterpret_cast<u32x4*>(k_lds + kr * 128 + ((ck ^ (kr & 7)) << 4)) = kreg[it];
      const int vr = (item & 15) + 16 * (item >> 7);
      const int vc = ((item >> 4) & 3) + 4 * ((item >> 6) & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vt_lds[(vc * 8 + e) * vld + vr] = static_cast<bf16>((vreg[it][e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
  }
  __syncthreads();

  bf16* obase = static_cast<bf16*>(p.o) + (long long)n * B * p.ldo + h * kDh;
#pragma unroll
  for (int ti = 0; ti < kTilesPerWave; ++ti) {
    const int tile = wave + 4 * ti;
    if (tile >= KT) break;
    const bf16x8_t* const qf = qall[ti];
    // S^T[key][q]: lane holds keys 16 kt + 4 g + r of query ql
    f32x4_t st[kKT2];
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < kKT2; ++kt) {
      st[kt] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (kt < KT) {
        const int kr = kt * 16 + ql;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
              k_lds + kr * 128 + (((4 * s + g) ^ (kr & 7)) << 4));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // only the last key tile can hold padding keys; scores stay unscaled
          // here (the scale is positive, so it commutes with the max)
          const float v = (kt < KT - 1 || kt * 16 + 4 * g + r < B) ? acc[r] : -INFINITY;
          st[kt][r] = v;
          bmax = fmaxf(bmax, v);
        }
      }
      // bound how many K fragments the scheduler keeps in flight (register pressure)
      if ((kt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    // p = exp((s - max) scale) = 2^(s sl2 - max sl2): one fma per score
    const float nmax = -wave_max_q(bmax) * sl2;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < kKT2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(st[kt][r], sl2, nmax));
        st[kt][r] = e;
        psum += e;
      }
    // O^T[dh][q] = V^T[dh][key] P^T[key][q]; MFMA k-slot 8 g + e stands for key
    // 32 sg + 4 g + e (e < 4) or 32 sg + 16 + 4 g + (e - 4) (e >= 4)
    f32x4_t oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sg = 0; sg < kKT2 / 2; ++sg) {
      union { uint32_t u[4]; bf16x8_t v; } pf;
      pf.u[0] = pack_bf16x2(st[2 * sg][0], st[2 * sg][1]);
      pf.u[1] = pack_bf16x2(st[2 * sg][2], st[2 * sg][3]);
      pf.u[2] = pack_bf16x2(st[2 * sg + 1][0], st[2 * sg + 1][1]);
      pf.u[3] = pack_bf16x2(st[2 * sg + 1][2], st[2 * sg + 1][3]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16* vrow = vt_lds + (dt * 16 + ql) * vld + 32 * sg + 4 * g;
        union { uint2 u[2]; bf16x8_t v; } vf;
        vf.u[0] = *reinterpret_cast<const uint2*>(vrow);
        vf.u[1] = *reinterpret_cast<const uint2*>(vrow + 16);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pf.v, oacc[dt], 0, 0, 0);
      }
    }
    // lane holds O[q = 16 tile + ql][dh = 16 dt + 4 g + r]
    const float inv = 1.0f / wave_sum_q(psum);
    const int q = tile * 16 + ql;
    if (q < B) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        uint2 u;
        u.x = pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv);
        u.y = pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv);
        *reinterpret_cast<uint2*>(obase + (long long)q * p.ldo + dt * 16 + 4 * g) = u;
      }
    }
  }
}

// Several frame blocks (KV cache): an online (running max / sum) softmax over
// 64-key groups, rescaling the O accumulators whenever the max grows.
__global__ __launch_bounds__(256) void attn_bf16_multi_kernel(AttnArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int B = p.B, kpad = kpad_of(B), vld = vt_ld_of(B);
  uint8_t* k_lds = lds;
  bf16* vt_lds = reinterpret_cast<bf16*>(lds + kpad * kDh * 2);

  const int n = blockIdx.x / p.heads, h = blockIdx.x % p.heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q_tiles = (B + 15) / 16;
  const int g = lane >> 4, ql = lane & 15;
  const float sl2 = p.scale * 1.4426950408889634f;   // softmax in base 2

  const bf16* qbase = static_cast<const bf16*>(p.q) + (long long)n * B * p.ldq + h * kDh;

  // per query tile: Q fragments (B operand of S^T = K Q^T), running max / sum, O^T accumulators
  bf16x8_t qf[kMaxTilesPerWave][2];
  float mrun[kMaxTilesPerWave], lrun[kMaxTilesPerWave];
  f32x4_t oacc[kMaxTilesPerWave][4];
#pragma unroll
  for (int ti = 0; ti < kMaxTilesPerWave; ++ti) {
    const int tile = wave + 4 * ti;
    const int qr = min(tile * 16 + ql, B - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qf[ti][s] = *reinterpret_cast<const bf16x8_t*>(qbase + (long long)qr * p.ldq + 32 * s + 8 * g);
    mrun[ti] = -INFINITY;
    lrun[ti] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[ti][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int blk = 0; blk < p.nblk; ++blk) {
    const bf16* kvb = static_cast<const bf16*>(p.kv[blk]) + (long long)n * B * p.ldkv + h * kDh;
    // ---- K: 8 lanes per 128-byte key row (coalesced), 16-byte swizzled LDS stores
    for (int item = tid; item < kpad * 8; item += 256) {
      const int kr = item >> 3, ck = item & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(kvb + (long long)min(kr, B - 1) * p.ldkv + ck * 8);
      *reinterpret_cast<uint4*>(k_lds + kr * 128 + ((ck ^ (kr & 7)) << 4)) = v;
    }
    // ---- V: a wave takes 16 keys x 4 chunks, so each transposed 2-byte store
    // instruction writes 4 Vt rows x 32 contiguous bytes on distinct banks
    for (int item = tid; item < kpad * 8; item += 256) {
      const int kr = (item & 15) + 16 * (item >> 7);
      const int ck = ((item >> 4) & 3) + 4 * ((item >> 6) & 1);
      const uint4 v = *reinterpret_cast<const uint4*>(kvb + p.d + (long long)min(kr, B - 1) * p.ldkv + ck * 8);
      const bf16* ve = reinterpret_cast<const bf16*>(&v);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt_lds[(ck * 8 + e) * vld + kr] = ve[e];
    }
    __syncthreads();

#pragma unroll
    for (int ti = 0; ti < kMaxTilesPerWave; ++ti) {
      const int tile = wave + 4 * ti;
      if (tile >= q_tiles) break;
      for (int g0 = 0; g0 < kpad; g0 += 64) {
        const int nkt = min(4, (kpad - g0) >> 4);   // 4, or 2 in a trailing 32-key group
        const int valid = B - g0;                   // keys >= valid are padding
        // S^T[key][q]: lane holds keys g0 + 16 kt + 4 g + r of query ql
        f32x4_t st[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (kt < nkt) {
            const int kr = g0 + kt * 16 + ql;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
                  k_lds + kr * 128 + (((4 * s + g) ^ (kr & 7)) << 4));
              st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ti][s], st[kt], 0, 0, 0);
            }
          }
        }
        float cmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kt * 16 + 4 * g + r;
            const float v = (kt < nkt && key < valid) ? st[kt][r] * sl2 : -INFINITY;
            st[kt][r] = v;
            cmax = fmaxf(cmax, v);
          }
        cmax = wave_max_q(cmax);
        const float mnew = fmaxf(mrun[ti], cmax);      // finite: every group has a valid key
        const float alpha = exp2f(mrun[ti] - mnew);    // exp2(-inf) = 0 on the first group
        mrun[ti] = mnew;
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = exp2f(st[kt][r] - mnew);
            st[kt][r] = e;
            psum += e;
          }
        lrun[ti] = lrun[ti] * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[ti][dt] *= alpha;
        // O^T[dh][q] += V^T[dh][key] P^T[key][q]; MFMA k-slot 8 g + e stands for key
        // g0 + 32 sg + 4 g + e (e < 4) or g0 + 32 sg + 16 + 4 g + (e - 4) (e >= 4)
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
          if (2 * sg < nkt) {
            union { uint32_t u[4]; bf16x8_t v; } pf;
            pf.u[0] = pack_bf16x2(st[2 * sg][0], st[2 * sg][1]);
            pf.u[1] = pack_bf16x2(st[2 * sg][2], st[2 * sg][3]);
            pf.u[2] = pack_bf16x2(st[2 * sg + 1][0], st[2 * sg + 1][1]);
            pf.u[3] = pack_bf16x2(st[2 * sg + 1][2], st[2 * sg + 1][3]);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              const bf16* vrow = vt_lds + (dt * 16 + ql) * vld + g0 + 32 * sg + 4 * g;
              union { uint2 u[2]; bf16x8_t v; } vf;
              vf.u[0] = *reinterpret_cast<const uint2*>(vrow);
              vf.u[1] = *reinterpret_cast<const uint2*>(vrow + 16);
              oacc[ti][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pf.v, oacc[ti][dt], 0, 0, 0);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // lane holds O[q = 16 tile + ql][dh = 16 dt + 4 g + r]
  bf16* obase = static_cast<bf16*>(p.o) + (long long)n * B * p.ldo + h * kDh;
#pragma unroll
  for (int ti = 0; ti < kMaxTilesPerWave; ++ti) {
    const int tile = wave + 4 * ti;
    if (tile >= q_tiles) break;
    const float inv = 1.0f / wave_sum_q(lrun[ti]);
    const int q = tile * 16 + ql;
    if (q < B) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        uint2 u;
        u.x = pack_bf16x2(oacc[ti][dt][0] * inv, oacc[ti][dt][1] * inv);
        u.y = pack_bf16x2(oacc[ti][dt][2] * inv, oacc[ti][dt][3] * inv);
        *reinterpret_cast<uint2*>(obase + (long long)q * p.ldo + dt * 16 + 4 * g) = u;
      }
    }
  }
}

// fp32: one thread per query row, keys streamed from global memory with an
// online softmax in fp32 (expf).  Used by fp32 models (small shapes).
template <int DH>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs p) {
  const int n = blockIdx.x / p.heads, h = blockIdx.x % p.heads;
  const int B = p.B;
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const float* qr = static_cast<const float*>(p.q) + ((long long)n * B + i) * p.ldq + h * DH;
    float q[DH], o[DH];
#pragma unroll
    for (int j = 0; j < DH; ++j) { q[j] = qr[j]; o[j] = 0.f; }
    float m = -INFINITY, l = 0.f;
    for (int blk = 0; blk < p.nblk; ++blk) {
      const float* kvb = static_cast<const float*>(p.kv[blk]);
      for (int r = 0; r < B; ++r) {
        const float* kr = kvb + ((long long)n * B + r) * p.ldkv + h * DH;
        const float* vr = kr + p.d;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < DH; ++j) s = fmaf(q[j], kr[j], s);
        s *= p.scale;
        const float mn = fmaxf(m, s);
        const float a = expf(m - mn), e = expf(s - mn);
        l = l * a + e;
#pragma unroll
        for (int j = 0; j < DH; ++j) o[j] = o[j] * a + e * vr[j];
        m = mn;
      }
    }
    float* orow = static_cast<float*>(p.o) + ((long long)n * B + i) * p.ldo + h * DH;
    const float inv = 1.0f / l;
#pragma unroll
    for (int j = 0; j < DH; ++j) orow[j] = o[j] * inv;
  }
}

}  // namespace

bool attention_bf16_supports(int dh, int B) {
  return dh == kDh && B >= 1 && B <= 16 * 4 * kMaxTilesPerWave;
}
bool attention_f32_supports(int dh) { return dh == 16 || dh == 32 || dh == 64 || dh == 128; }

template <int KT>
hipError_t set_lds_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_single_kernel<KT>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes_of(16 * KT));
}
template <int... KTs>
hipError_t set_all(std::integer_sequence<int, KTs...>) {
  hipError_t e = hipSuccess;
  ((e = (e == hipSuccess ? set_lds_attr<KTs + 1>() : e)), ...);
  return e;
}
template <int... KTs>
void launch_kt(int kt, const AttnArgs& a, hipStream_t stream, std::integer_sequence<int, KTs...>) {
  ((kt == KTs + 1 ? (attn_bf16_single_kernel<KTs + 1><<<a.n * a.heads, 256, lds_bytes_of(a.B), stream>>>(a), 0) : 0), ...);
}
using KtRange = std::make_integer_sequence<int, kMaxKeyTiles>;

hipError_t attention_init() {
  const hipError_t e = set_all(KtRange{});
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_multi_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes_of(16 * kMaxKeyTiles));
}

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const int kt = (a.B + 15) / 16;
  if (kt < 1 || kt > kMaxKeyTiles) return hipErrorInvalidValue;
  if (a.nblk == 1)
    launch_kt(kt, a, stream, KtRange{});
  else
    attn_bf16_multi_kernel<<<a.n * a.heads, 256, lds_bytes_of(a.B), stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const int grid = a.n * a.heads;
  switch (a.dh) {
    case 16: attn_f32_kernel<16><<<grid, 128, 0, stream>>>(a); break;
    case 32: attn_f32_kernel<32><<<grid, 128, 0, stream>>>(a); break;
    case 64: attn_f32_kernel<64><<<grid, 128, 0, stream>>>(a); break;
    case 128: attn_f32_kernel<128><<<grid, 128, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cem
