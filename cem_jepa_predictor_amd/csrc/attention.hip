// Block-causal multi-head attention of the predictor's current frame block.
//
// Page "Real-Time Inference for JEPA World Model Architectures with Ray",
// section 05: the predictor is frame-causal, so at rollout step t the queries
// of frame block t attend to the keys of blocks 0..t, and the keys/values of
// earlier blocks come from a KV cache instead of being recomputed.  Within a
// block attention is bidirectional.  Softmax scale 1/sqrt(dh), fp32 softmax.
//
// bf16 kernels (dh = 64), one workgroup per (candidate, head).
//
// One frame block (the whole plan at horizon 1): 512 threads (8 waves), two
// workgroups per CU, so each SIMD holds four waves.
//  * K and V rows of the block (B keys, padded to a multiple of 32 with zero
//    rows) go global -> LDS by buffer_load ... lds, both row-major with 16-byte
//    chunks XOR-swizzled by key % 8: 74 KB.  Q fragments go straight to
//    registers, one query tile ahead.
//  * Each wave owns 16-row query tiles.  S^T = K Q^T with
//    v_mfma_f32_16x16x32_bf16 (lane l holds the scores of query l % 16), in two
//    key halves joined by one online-softmax rescale, so only half a row of
//    scores is live in registers; exact max per half, one fma + exp2 per score.
//  * O^T += V^T P^T with P taken straight from registers: the MFMA sums over
//    its 32 key slots, and the key each slot stands for is chosen so the lane's
//    own probabilities and the matching V^T entries line up.  V^T fragments
//    come from the row-major V through gfx950's transposing LDS read
//    (ds_read_b64_tr_b16): lane 16 g + 4 r + c reads 4 dh-values of key r,
//    lane 16 g + i receives 4 keys of dh-row i.
//  * HBM traffic per (candidate, head) is one read of Q, K, V and one write of
//    O.  At the V-JEPA2-AC shape that traffic alone would take about 0.2 ms
//    per launch; the kernel takes about twice that, with neither the vector
//    ALUs nor the matrix cores saturated: its dependency chains (scores ->
//    max -> exp2 -> P V) at four waves per SIMD, and the K/V staging of each
//    workgroup, set the pace.  exp2 issues at the rate of an fma here.
//
// Several frame blocks (KV cache, horizon > 1): the same 512-thread structure
// with the blocks streamed through LDS one at a time and, per query tile, the
// online-softmax state carried across blocks in registers.
//
// Layer 0 of the first frame block at horizon 1 reads q, k and v through a row
// index instead (AttnArgs::qkv_c): each candidate's action row and its problem's
// shared state and frame rows, projected once each into one compact block.
#include <type_traits>
#include <utility>

#include "kernels.hpp"

namespace cem {
namespace {

constexpr int kDh = 64;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t* lds_v4bf16_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kMaxKeyTiles = 20;     // 16-key tiles per frame block -> B <= 320

constexpr __host__ __device__ int kpad_of(int B) { return (B + 31) & ~31; }
// K and V of one frame block, row-major, padded to a multiple of 32 keys
__host__ __device__ __forceinline__ int lds_bytes_of(int B) { return 2 * kpad_of(B) * kDh * 2; }

// Lanes l, l^16, l^32, l^48 share query l % 16.  v_permlane16_swap exchanges the
// odd 16-lane rows of its first operand with the even rows of its second: with
// both operands v, the two results hold (v[l], v[l ^ 16]) in some order in every
// lane, so their max or sum is the xor-16 combination; v_permlane32_swap does the
// same for the two 32-lane halves.  Plain VALU: no LDS round trip.
__device__ __forceinline__ float wave_max_q(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_q(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One frame block (every query sees exactly the B keys of its own block).
// 512 threads (8 waves) per (candidate, head); two workgroups share a CU, so
// each SIMD holds four waves whose dependency chains (scores -> max -> exp ->
// P V) hide one another.  K and V go global -> LDS by buffer_load ... lds
// (rows past B read as zero).  Each wave owns the 16-query tiles w, w + 8, ...;
// per tile the keys are taken in two halves with one online-softmax rescale
// between them, which keeps the score registers to one half.
// KT = ceil(B / 16): 16-key (and 16-query) tiles per block, fixed per model.
template <int KT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void attn_bf16_single_kernel(AttnArgs p) {
  constexpr int kKT2 = 2 * ((KT + 1) / 2);   // key tiles rounded up to MFMA k = 32 pairs
  constexpr int kSG = kKT2 / 2;              // 32-key groups
  constexpr int kSG0 = (kSG + 1) / 2;        // groups in the first half
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int B = p.B, kpad = kpad_of(B);
  uint8_t* k_lds = lds;
  uint8_t* v_lds = lds + kpad * kDh * 2;   // row-major like K (read transposed)

  const int n = blockIdx.x / p.heads, h = blockIdx.x % p.heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, ql = lane & 15;
  const int vr4 = (lane >> 2) & 3, vc4 = lane & 3;   // transposing-read source slot
  const float sl2 = p.scale * 1.4426950408889634f;   // softmax in base 2

  // Compact layer-0 source (AttnArgs::qkv_c): row r of this candidate is row crow(r) of
  // the compact q|k|v block (3 d wide): its action row after every problem's shared rows,
  // the shared rows of its problem otherwise.
  const bool cmp = p.qkv_c != nullptr;
  const int ldc = 3 * p.d;
  const int c_act = p.c_problems * (B - 1) + n;
  const int c_sh = cmp ? (n / p.c_n_per) * (B - 1) - 1 : 0;
  auto crow = [&](int r) { return r == 0 ? c_act : c_sh + r; };

  // ---- K and V rows 0 .. kpad-1 of this (candidate, head) -> LDS, 8 rows (1 KB) per
  // instruction; LDS row r holds 16-byte chunk c at c ^ (r & 7)
  {
    const int rows8 = kpad >> 3, ninstr = 2 * rows8;
    const int lrow = lane >> 3, lch = (lane & 7) ^ (lane >> 3);
    if (cmp) {
      // rows past B take an offset beyond the resource: they read as zero
      const bf16* kb = static_cast<const bf16*>(p.qkv_c) + p.d + h * kDh;
      const int bytes = (p.c_problems * (B - 1) + p.n - 1) * ldc * 2 + kDh * 2;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kb), (short)0, bytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kb + p.d), (short)0, bytes, 0x00020000);
      for (int t = wave; t < ninstr; t += 8) {
        const bool isv = t >= rows8;
        const int r0 = 8 * (isv ? t - rows8 : t), r = r0 + lrow;
        const int voff = r < B ? crow(r) * ldc * 2 + lch * 16 : 0x7ffffff0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (lds_ptr_t)((isv ? v_lds : k_lds) + r0 * 128), 16, voff, 0, 0, 0);
      }
    } else {
      const bf16* kvb = static_cast<const bf16*>(p.kv[0]) + (long long)n * B * p.ldkv + h * kDh;
      const int bytes = (B - 1) * p.ldkv * 2 + kDh * 2;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kvb), (short)0, bytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kvb + p.d), (short)0, bytes, 0x00020000);
      for (int t = wave; t < ninstr; t += 8) {
        const bool isv = t >= rows8;
        const int r0 = 8 * (isv ? t - rows8 : t);
        const int voff = (r0 + lrow) * p.ldkv * 2 + lch * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (lds_ptr_t)((isv ? v_lds : k_lds) + r0 * 128), 16, voff, 0, 0, 0);
      }
    }
  }
  const bf16* qbase = cmp ? static_cast<const bf16*>(p.qkv_c) + h * kDh
                          : static_cast<const bf16*>(p.q) + (long long)n * B * p.ldq + h * kDh;
  const int qld = cmp ? ldc : p.ldq;
  auto load_q = [&](int tile, bf16x8_t q[2]) {
    const int qi = min(tile * 16 + ql, B - 1);
    const int qr = cmp ? crow(qi) : qi;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      q[s] = *reinterpret_cast<const bf16x8_t*>(qbase + (long long)qr * qld + 32 * s + 8 * g);
  };
  bf16x8_t qf[2], qn[2];
  load_q(wave, qf);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's K/V rows and Q landed
  __syncthreads();

  bf16* obase = static_cast<bf16*>(p.o) + (long long)n * B * p.ldo + h * kDh;
  for (int tile = wave; tile < KT; tile += 8) {
    if (tile + 8 < KT) load_q(tile + 8, qn);
    f32x4_t oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    // one half: key groups [SG_A, SG_B)
    auto half = [&](auto sga, auto sgb) {
      constexpr int SGA = decltype(sga)::value, SGB = decltype(sgb)::value;
      constexpr int NT = 2 * (SGB - SGA);
      // S^T[key][q]: lane holds keys 16 kt + 4 g + r of query ql
      f32x4_t st[NT];
      float bmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int kt = 2 * SGA + i;
        st[i] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
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
            st[i][r] = v;
            bmax = fmaxf(bmax, v);
          }
        }
        // bound how many K fragments the scheduler keeps in flight (register pressure)
        if ((i & 1) == 1) __builtin_amdgcn_sched_barrier(0);
      }
      const float mnew = fmaxf(mrun, wave_max_q(bmax));   // finite: the first half has a valid key
      const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * sl2);   // 0 on the first half
      const float nmax = -mnew * sl2;
      mrun = mnew;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(st[i][r], sl2, nmax));
          st[i][r] = e;
          psum += e;
        }
      lrun = fmaf(lrun, alpha, psum);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
      // O^T[dh][q] += V^T[dh][key] P^T[key][q]; MFMA k-slot 8 g + e stands for key
      // 32 sg + 4 g + e (e < 4) or 32 sg + 16 + 4 g + (e - 4) (e >= 4)
#pragma unroll
      for (int j = 0; j < NT / 2; ++j) {
        const int sg = SGA + j;
        union { uint32_t u[4]; bf16x8_t v; } pf;
        pf.u[0] = pack_bf16x2(st[2 * j][0], st[2 * j][1]);
        pf.u[1] = pack_bf16x2(st[2 * j][2], st[2 * j][3]);
        pf.u[2] = pack_bf16x2(st[2 * j + 1][0], st[2 * j + 1][1]);
        pf.u[3] = pack_bf16x2(st[2 * j + 1][2], st[2 * j + 1][3]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          // V^T fragment through transposing reads: lane 16 g + 4 r + c fetches
          // V[key0 + r][16 dt + 4 c .. +3]; lane 16 g + i receives V[key0 + 0..3][16 dt + i]
          const int row0 = 32 * sg + 4 * g + vr4, c16 = 2 * dt + (vc4 >> 1);
          union { bf16x4_t hh[2]; bf16x8_t v; } vf;
          vf.hh[0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_v4bf16_t)(v_lds + row0 * 128 + ((c16 ^ (row0 & 7)) << 4) + (vc4 & 1) * 8));
          const int row1 = row0 + 16;
          vf.hh[1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_v4bf16_t)(v_lds + row1 * 128 + ((c16 ^ (row1 & 7)) << 4) + (vc4 & 1) * 8));
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pf.v, oacc[dt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    half(std::integral_constant<int, 0>{}, std::integral_constant<int, kSG0>{});
    if constexpr (kSG0 < kSG) half(std::integral_constant<int, kSG0>{}, std::integral_constant<int, kSG>{});
    // lane holds O[q = 16 tile + ql][dh = 16 dt + 4 g + r]
    const float inv = 1.0f / wave_sum_q(lrun);
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
    qf[0] = qn[0]; qf[1] = qn[1];
  }
}

// Several frame blocks (KV cache): the single-block structure with the frame
// blocks streamed through LDS one at a time.  Each wave keeps, for each of its
// query tiles, a running max, a lane-partial sum and the O^T accumulators
// across blocks (online softmax); keys of a block are taken in thirds so the
// scores of one third and the state of three tiles fit 128 VGPRs.
template <int KT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void attn_bf16_multi8_kernel(AttnArgs p) {
  constexpr int kKT2 = 2 * ((KT + 1) / 2);   // key tiles per block, rounded up to pairs
  constexpr int kSG = kKT2 / 2;              // 32-key groups per block
  constexpr int kTPW = (KT + 7) / 8;         // query tiles per wave (at most)
  constexpr int kP0 = (kSG + 2) / 3, kP1 = (kSG - kP0 + 1) / 2, kP2 = kSG - kP0 - kP1;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int B = p.B, kpad = kpad_of(B);
  uint8_t* k_lds = lds;
  uint8_t* v_lds = lds + kpad * kDh * 2;

  const int n = blockIdx.x / p.heads, h = blockIdx.x % p.heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, ql = lane & 15;
  const int vr4 = (lane >> 2) & 3, vc4 = lane & 3;
  const float sl2 = p.scale * 1.4426950408889634f;

  const bf16* qbase = static_cast<const bf16*>(p.q) + (long long)n * B * p.ldq + h * kDh;
  auto load_q = [&](int tile, bf16x8_t q[2]) {
    const int qr = min(tile * 16 + ql, B - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      q[s] = *reinterpret_cast<const bf16x8_t*>(qbase + (long long)qr * p.ldq + 32 * s + 8 * g);
  };
  auto keys = [&](auto ngc, int sg0, const bf16x8_t (&q)[2], f32x4_t (&oacc)[4], float& mrun, float& lrun) {
    constexpr int NG = decltype(ngc)::value, NT = 2 * NG;
    f32x4_t st[NT];
    float bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int kt = 2 * sg0 + i;
      st[i] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (kt < KT) {
        const int kr = kt * 16 + ql;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
              k_lds + kr * 128 + (((4 * s + g) ^ (kr & 7)) << 4));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, q[s], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = (kt < KT - 1 || kt * 16 + 4 * g + r < B) ? acc[r] : -INFINITY;
          st[i][r] = v;
          bmax = fmaxf(bmax, v);
        }
      }
      if ((i & 1) == 1) __builtin_amdgcn_sched_barrier(0);
    }
    // every key group holds a valid key, so mnew is finite and alpha = 0 on the first pass
    const float mnew = fmaxf(mrun, wave_max_q(bmax));
    const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * sl2);
    const float nmax = -mnew * sl2;
    mrun = mnew;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(st[i][r], sl2, nmax));
        st[i][r] = e;
        psum += e;
      }
    lrun = fmaf(lrun, alpha, psum);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int sg = sg0 + j;
      union { uint32_t u[4]; bf16x8_t v; } pf;
      pf.u[0] = pack_bf16x2(st[2 * j][0], st[2 * j][1]);
      pf.u[1] = pack_bf16x2(st[2 * j][2], st[2 * j][3]);
      pf.u[2] = pack_bf16x2(st[2 * j + 1][0], st[2 * j + 1][1]);
      pf.u[3] = pack_bf16x2(st[2 * j + 1][2], st[2 * j + 1][3]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int row0 = 32 * sg + 4 * g + vr4, c16 = 2 * dt + (vc4 >> 1);
        union { bf16x4_t hh[2]; bf16x8_t v; } vf;
        vf.hh[0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_v4bf16_t)(v_lds + row0 * 128 + ((c16 ^ (row0 & 7)) << 4) + (vc4 & 1) * 8));
        const int row1 = row0 + 16;
        vf.hh[1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_v4bf16_t)(v_lds + row1 * 128 + ((c16 ^ (row1 & 7)) << 4) + (vc4 & 1) * 8));
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.v, pf.v, oacc[dt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x4_t oacc[kTPW][4];
  float mrun[kTPW], lrun[kTPW];
#pragma unroll
  for (int ti = 0; ti < kTPW; ++ti) {
    mrun[ti] = -INFINITY;
    lrun[ti] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[ti][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int rows8 = kpad >> 3, ninstr = 2 * rows8;
  const int lrow = lane >> 3, lch = (lane & 7) ^ (lane >> 3);
  const int bytes = (B - 1) * p.ldkv * 2 + kDh * 2;
  for (int blk = 0; blk < p.nblk; ++blk) {
    if (blk > 0) __syncthreads();   // every wave is done with the previous block's K and V
    {
      const bf16* kvb = static_cast<const bf16*>(p.kv[blk]) + (long long)n * B * p.ldkv + h * kDh;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kvb), (short)0, bytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kvb + p.d), (short)0, bytes, 0x00020000);
      for (int t = wave; t < ninstr; t += 8) {
        const bool isv = t >= rows8;
        const int r0 = 8 * (isv ? t - rows8 : t);
        const int voff = (r0 + lrow) * p.ldkv * 2 + lch * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (lds_ptr_t)((isv ? v_lds : k_lds) + r0 * 128), 16, voff, 0, 0, 0);
      }
    }
    bf16x8_t qf[2];
    load_q(wave, qf);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's K/V rows and Q landed
    __syncthreads();
#pragma unroll
    for (int ti = 0; ti < kTPW; ++ti) {
      const int tile = wave + 8 * ti;
      if (tile < KT) {
        bf16x8_t qn[2];
        if (ti + 1 < kTPW && tile + 8 < KT) load_q(tile + 8, qn);
        keys(std::integral_constant<int, kP0>{}, 0, qf, oacc[ti], mrun[ti], lrun[ti]);
        if constexpr (kP1 > 0) keys(std::integral_constant<int, kP1>{}, kP0, qf, oacc[ti], mrun[ti], lrun[ti]);
        if constexpr (kP2 > 0) keys(std::integral_constant<int, kP2>{}, kP0 + kP1, qf, oacc[ti], mrun[ti], lrun[ti]);
        if (ti + 1 < kTPW && tile + 8 < KT) { qf[0] = qn[0]; qf[1] = qn[1]; }
      }
    }
  }
  bf16* obase = static_cast<bf16*>(p.o) + (long long)n * B * p.ldo + h * kDh;
#pragma unroll
  for (int ti = 0; ti < kTPW; ++ti) {
    const int tile = wave + 8 * ti;
    if (tile < KT) {
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
  return dh == kDh && B >= 1 && B <= 16 * kMaxKeyTiles;
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
void launch_multi_kt(int kt, const AttnArgs& a, hipStream_t stream, std::integer_sequence<int, KTs...>) {
  ((kt == KTs + 1 ? (attn_bf16_multi8_kernel<KTs + 1><<<a.n * a.heads, 512, lds_bytes_of(a.B), stream>>>(a), 0) : 0), ...);
}
template <int KT>
hipError_t set_multi_lds_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_multi8_kernel<KT>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes_of(16 * KT));
}
template <int... KTs>
hipError_t set_all_multi(std::integer_sequence<int, KTs...>) {
  hipError_t e = hipSuccess;
  ((e = (e == hipSuccess ? set_multi_lds_attr<KTs + 1>() : e)), ...);
  return e;
}
template <int... KTs>
void launch_kt(int kt, const AttnArgs& a, hipStream_t stream, std::integer_sequence<int, KTs...>) {
  ((kt == KTs + 1 ? (attn_bf16_single_kernel<KTs + 1><<<a.n * a.heads, 512, lds_bytes_of(a.B), stream>>>(a), 0) : 0), ...);
}
using KtRange = std::make_integer_sequence<int, kMaxKeyTiles>;

hipError_t attention_init() {
  hipError_t e = set_all(KtRange{});
  if (e != hipSuccess) return e;
  return set_all_multi(KtRange{});
}

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const int kt = (a.B + 15) / 16;
  if (kt < 1 || kt > kMaxKeyTiles) return hipErrorInvalidValue;
  if (a.qkv_c && (a.nblk != 1 || a.B < 2 || a.c_problems <= 0 || a.c_n_per <= 0 ||
                  a.n != a.c_problems * a.c_n_per ||
                  ((long long)a.c_problems * (a.B - 1) + a.n) * 3 * a.d * 2 >= 0x7ffffff0LL))
    return hipErrorInvalidValue;
  if (a.nblk == 1)
    launch_kt(kt, a, stream, KtRange{});
  else
    launch_multi_kt(kt, a, stream, KtRange{});
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
