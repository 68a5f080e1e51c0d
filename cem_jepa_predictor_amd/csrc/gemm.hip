// Dense projections of the predictor: out = epilogue(A[M, K] @ Bt[N, K]^T).
//
// Every linear layer of the action-conditioned predictor (fused q|k|v, output
// projection, MLP up with GELU, MLP down, frame in/out projections) goes
// through here.  These GEMMs carry about 95% of the plan step's FLOPs at the
// V-JEPA2-AC predictor shape (page "Real-Time Inference for JEPA World Model
// Architectures with Ray", section 01: ~8,000 predictor evaluations per
// action), so the bf16 kernel is MFMA-bound by design.
//
// bf16 kernel (gfx950):
//  * 256 x 256 output tile per 256-thread workgroup, BK = 64; four wave64s in
//    a 2 x 2 grid, each owning a 128 x 128 sub-tile = 4 x 4 tiles of
//    v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane).
//  * The MFMA's first operand is the weight tile and its second the
//    activation tile, so each lane's accumulator quads hold 4 consecutive
//    output columns of one output row.
//  * Operands: global -> VGPR (buffer_load_dwordx4, two staging register sets)
//    -> LDS double buffer (2 x 64 KB), memory two slabs ahead of the MFMAs,
//    every memory instruction placed between MFMAs (see the main loop).
//    128-byte LDS rows hold their eight 16-byte chunks at c ^ ((r >> 1) & 7),
//    so fragment reads are free of bank conflicts.
//  * Block -> tile map is XCD-aware: the dispatcher hands block b to XCD
//    b % 8, so each XCD receives a contiguous range of logical tiles, ordered
//    in groups of 8 row-tiles to share A and B panels in that XCD's L2.
//  * Ragged M / N: operand loads go through buffer resources bounded at the
//    tile's last valid row (the hardware returns zero beyond it), stores are
//    masked.
//  * Results leave through LDS as full rows (see the epilogue).
//  * One kernel instantiation per epilogue kind (plain, GELU, residual), so
//    each carries only its own epilogue code.
//
// Epilogue (fp32): + bias, optional GELU, optional residual add (the
// output already holds the residual stream), optional column split into two
// destinations (q -> Q buffer, k|v -> KV cache), optional output-row remap.
#include "kernels.hpp"

namespace cem {
namespace {

// ------------------------------------------------------------------ epilogue
template <typename T> struct Store4;
template <> struct Store4<bf16> {
  __device__ static __forceinline__ void load(const bf16* p, float v[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  }
  __device__ static __forceinline__ void store(bf16* p, const float v[4]) {
    uint2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = u;
  }
  __device__ static __forceinline__ float gelu(float x) { return gelu_bf16_path(x); }
};
template <> struct Store4<float> {
  __device__ static __forceinline__ void load(const float* p, float v[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  __device__ static __forceinline__ void store(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ static __forceinline__ float gelu(float x) { return gelu_exact(x); }
};

// Four consecutive output columns n..n+3 (n % 4 == 0, N % 4 == 0) of the
// physical output row `row`.
enum { kEpiPlain = 0, kEpiGelu = 1, kEpiResidual = 2 };

template <typename T, int KIND>
__device__ __forceinline__ void epilogue_row4(const Epilogue& e, int N, long long row, int n,
                                              float v[4]) {
  if (n >= N) return;
  if (e.bias) {
    const float4 bb = *reinterpret_cast<const float4*>(e.bias + n);
    v[0] += bb.x; v[1] += bb.y; v[2] += bb.z; v[3] += bb.w;
  }
  if constexpr (KIND == kEpiGelu) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = Store4<T>::gelu(v[i]);
  }
  T* p = (n < e.split) ? static_cast<T*>(e.c0) + row * e.ld0 + n
                       : static_cast<T*>(e.c1) + row * e.ld1 + (n - e.split);
  if constexpr (KIND == kEpiResidual) {
    float r[4];
    Store4<T>::load(p, r);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += r[i];
  }
  Store4<T>::store(p, v);
}

// ------------------------------------------------------------------ bf16 MFMA kernel
constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int TILE_BYTES = BM * BK * 2;       // 32 KB per operand slab
constexpr int STAGE_BYTES = 2 * TILE_BYTES;   // A slab + B slab
constexpr int GROUP_M = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void tile_of_block(int b, int nb, int tiles_m, int tiles_n, int& tm,
                                              int& tn) {
  const int xcd = b & 7, slot = b >> 3;
  const int base = nb >> 3, rem = nb & 7;
  const int L = xcd * base + min(xcd, rem) + slot;
  const int per_group = GROUP_M * tiles_n;
  const int g = L / per_group;
  const int first_m = g * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in = L - g * per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// Buffer resource over rows [row0, row0 + rows) of a row-major bf16 matrix,
// advanced by k elements; loads past the last valid row return zero.
// Valid rows stay in range for every k < K <= ld: r * ld * 2 + 2k + 16 <= rows * ld * 2.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const bf16* base, int row0, int rows,
                                                            int ld, int k) {
  const uint32_t bytes = (uint32_t)rows * (uint32_t)ld * 2u - (uint32_t)k * 2u;
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(base + (long long)row0 * ld + k), (short)0, (int)bytes, 0x00020000);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Main loop.  Operand slabs (BK = 64 columns of 256 A rows and 256 B rows,
// 128 contiguous bytes per row) go global -> VGPR -> LDS through two staging
// register sets, so memory runs two slabs ahead of the MFMAs without a third
// LDS stage: during slab kt the wave issues slab kt+2's loads (4 per substep)
// and writes slab kt+1 (loaded during slab kt-1) into the free LDS stage
// (substeps 0-2), each interleaved one per MFMA so no burst of memory
// instructions holds up MFMA issue.  One barrier per slab, before the last
// substep's MFMAs; it waits for LDS traffic only.  Loads of slabs at or past K
// use an empty buffer resource (zeros, no memory traffic), which keeps every
// slab of the loop identical; an odd slab count runs one extra all-zero slab.
//
// Epilogue.  When a tile maps to one destination with 16-byte aligned rows,
// each wave stages its 128 x 128 result in 32 KB of the freed operand LDS and
// then writes full rows (16 bytes a lane, 4 rows x 256 bytes per
// instruction) instead of 16-byte pieces of 32 rows.  Plain / GELU values are
// staged as bf16 (rounded once, as before); the residual kind stages fp32 in
// two 64-row halves and adds the residual rows, loaded first, in fp32, so it
// also rounds once.  Other tiles take the per-4-column path.
template <int KIND>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(const bf16* __restrict__ A, int lda,
                                                         const bf16* __restrict__ Bt, int ldb,
                                                         int M, int N, int K, Epilogue epi) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) float bias_lds[BN];   // this tile's bias columns
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);

  // Global loads: wave instruction j covers rows 8 (4 j + wave) .. +7 of an operand
  // slab, lane l row + l / 8, logical 16-byte chunk l % 8.  LDS row r holds its
  // logical chunk c at position c ^ ((r >> 1) & 7): a b128 fragment read is served
  // 16 lanes (rows r..r+15) per pass over 64 four-byte banks, and (row parity,
  // (r >> 1) & 7) gives those 16 rows 16 distinct bank groups.  Rows
  // 8 (4 j + wave) + lrow have (r >> 1) & 7 = (4 (wave & 1) + (lrow >> 1)) & 7.
  const int lrow = lane >> 3, lc = lane & 7;
  const int sw = (4 * (wave & 1) + (lrow >> 1)) & 7;
  const int goff_a = (8 * wave + lrow) * lda * 2 + lc * 16, gstep_a = 32 * lda * 2;
  const int goff_b = (8 * wave + lrow) * ldb * 2 + lc * 16, gstep_b = 32 * ldb * 2;
  const int lds_w = (8 * wave + lrow) * 128 + ((lc ^ sw) << 4);
  const int KT = K / BK;
  // part p < 8: A rows of instruction p; p >= 8: B rows of instruction p - 8.
  // The row offset stays in the range-checked VGPR offset (soffset is not checked).
  auto gload = [&](u32x4* g, int kt, int p0, int p1) {
    const bool live = kt < KT;
    const __amdgpu_buffer_rsrc_t ra = slab_rsrc(A, m0, live ? rows_a : 0, lda, live ? kt * BK : 0);
    const __amdgpu_buffer_rsrc_t rb = slab_rsrc(Bt, n0, live ? rows_b : 0, ldb, live ? kt * BK : 0);
#pragma unroll
    for (int p = p0; p < p1; ++p) {
      const int j = p & 7;
      g[p] = (p < 8) ? __builtin_amdgcn_raw_buffer_load_b128(ra, goff_a + j * gstep_a, 0, 0)
                     : __builtin_amdgcn_raw_buffer_load_b128(rb, goff_b + j * gstep_b, 0, 0);
    }
  };
  auto lstore = [&](const u32x4* g, uint8_t* stage, int p0, int p1) {
#pragma unroll
    for (int p = p0; p < p1; ++p)
      *reinterpret_cast<u32x4*>(stage + (p < 8 ? 0 : TILE_BYTES) + lds_w + (p & 7) * 4096) = g[p];
  };

  // fragments: lane reads row (l % 32) of a 32-row MFMA tile, k half (l / 32)
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fk = lane >> 5;
  const int arow = (wm * 128 + fr) * 128;
  const int brow = TILE_BYTES + (wn * 128 + fr) * 128;
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8_t fa[2][4], fb[2][4];
  auto frags = [&](const uint8_t* stage, int s, int buf) {
    const int pc = ((2 * s + fk) ^ ((fr >> 1) & 7)) << 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[buf][i] = *reinterpret_cast<const bf16x8_t*>(stage + arow + i * 4096 + pc);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[buf][j] = *reinterpret_cast<const bf16x8_t*>(stage + brow + j * 4096 + pc);
  };
  // The weight tile is the MFMA's first operand, so D[i][j] has j = output row
  // (lane % 32) and i = output column 8 (r / 4) + 4 (lane / 32) + r % 4.
  auto mfma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };
  auto lds_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); global loads stay in flight
    __builtin_amdgcn_s_barrier();
  };
  // schedule of one substep: its 8 fragment reads first, then one LDS write and one
  // global load after each of the first nw / nl MFMAs
  auto interleave = [&](int nw, int nl) {
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    for (int r = 0; r < 16; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (r < nw) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      if (r < nl) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };
#define CEM_FENCE __builtin_amdgcn_sched_barrier(0)
  // One K-slab from `cur`: gw holds slab kt+1 (written to `nxt`), gl receives slab kt+2.
  auto slab = [&](uint8_t* cur, uint8_t* nxt, u32x4* gw, u32x4* gl, int kt) {
    frags(cur, 1, 1); lstore(gw, nxt, 0, 6); gload(gl, kt + 2, 0, 4); mfma(0); interleave(6, 4);
    CEM_FENCE;
    frags(cur, 2, 0); lstore(gw, nxt, 6, 11); gload(gl, kt + 2, 4, 8); mfma(1); interleave(5, 4);
    CEM_FENCE;
    frags(cur, 3, 1); lstore(gw, nxt, 11, 16); gload(gl, kt + 2, 8, 12); mfma(0); interleave(5, 4);
    CEM_FENCE;
    lds_barrier();
    frags(nxt, 0, 0); gload(gl, kt + 2, 12, 16); mfma(1); interleave(0, 4);
    CEM_FENCE;
  };
  // prologue: slabs 0 and 1 in flight together; slab 0 goes to LDS as it lands
  u32x4 g0[16], g1[16];
  gload(g0, 0, 0, 16);
  gload(g1, 1, 0, 16);
  // the tile's bias columns go to LDS once, so the epilogue reads them at LDS latency
  if (epi.bias && tid < BN / 4 && n0 + 4 * tid < N)
    *reinterpret_cast<float4*>(bias_lds + 4 * tid) = *reinterpret_cast<const float4*>(epi.bias + n0 + 4 * tid);
  CEM_FENCE;
  lstore(g0, st0, 0, 16);
  CEM_FENCE;
  lds_barrier();
  frags(st0, 0, 0);
  // The accumulators start at the bias (each lane's quads are 4 consecutive
  // output columns), so no epilogue adds it.  Columns past N are never stored.
  if (epi.bias) {
    const float* const bl = bias_lds + wn * 128 + 4 * fk;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 bb = *reinterpret_cast<const float4*>(bl + j * 32 + 8 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i][j][4 * q] = bb.x; acc[i][j][4 * q + 1] = bb.y;
          acc[i][j][4 * q + 2] = bb.z; acc[i][j][4 * q + 3] = bb.w;
        }
      }
  }
  CEM_FENCE;
  for (int kt = 0; kt < KT; kt += 2) {
    slab(st0, st1, g1, g0, kt);       // slab kt+1 from g1 into st1; slab kt+2 loads into g0
    slab(st1, st0, g0, g1, kt + 1);
  }
#undef CEM_FENCE

  const int ncol = n0 + wn * 128 + 4 * fk;
  const bool to_c0 = n0 + BN <= epi.split, to_c1 = n0 >= epi.split;
  bf16* const cbase = static_cast<bf16*>(to_c0 ? epi.c0 : epi.c1);
  const int ldc = to_c0 ? epi.ld0 : epi.ld1;
  const int cshift = to_c0 ? 0 : epi.split;
  if ((to_c0 || to_c1) && n0 + BN <= N && epi.bias && (ldc & 7) == 0 && (cshift & 7) == 0 &&
      epi.rows.group >= 4 && ((uintptr_t)cbase & 15) == 0) {
    // No barrier: after the last slab's barrier the operand stages see only
    // fragment reads whose values are never used, and each wave stages into its
    // own 32 KB, so a wave starts its epilogue as soon as its MFMAs are issued.
    uint8_t* const ep = (wave < 2 ? st0 : st1) + (wave & 1) * 32768;
    bf16* const cwave = cbase + (n0 + wn * 128 - cshift);
    const int row_base = m0 + wm * 128;
    // destination rows of one lane, advanced incrementally (row map group >= 4)
    struct RowWalk {
      long long quot;
      int rem;
    };
    auto row_walk = [&](int r) {
      const int m = row_base + r;
      return RowWalk{(long long)(m / epi.rows.group), m % epi.rows.group};
    };
    auto row_of = [&](const RowWalk& w) { return w.quot * epi.rows.stride + epi.rows.offset + w.rem; };
    auto row_step = [&](RowWalk& w, int d) {
      w.rem += d;
      if (w.rem >= epi.rows.group) { w.rem -= epi.rows.group; ++w.quot; }
    };
    // a row map whose group exceeds M sends row m to m + offset
    const bool plain_rows = epi.rows.group > M;
    if constexpr (KIND != kEpiResidual) {
      // bf16 staging: row r (256 bytes) holds 16-byte chunk c at c ^ (r & 15)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 32 + fr;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]};
            if constexpr (KIND == kEpiGelu) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = gelu_bf16_path(v[e]);
            }
            uint2 u;
            u.x = pack_bf16x2(v[0], v[1]);
            u.y = pack_bf16x2(v[2], v[3]);
            const int c16 = 4 * j + q;
            *reinterpret_cast<uint2*>(ep + r * 256 + ((c16 ^ (r & 15)) << 4) + fk * 8) = u;
          }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's staging writes are done
      const int c16 = lane & 15;
      auto store_rows = [&](auto row_ptr) {
        // all 32 row pieces come out of LDS first, so the stores issue back to back
        u32x4 d[32];
#pragma unroll
        for (int t = 0; t < 32; ++t) {
          const int r = 4 * t + (lane >> 4);
          d[t] = *reinterpret_cast<const u32x4*>(ep + r * 256 + ((c16 ^ (r & 15)) << 4));
        }
#pragma unroll
        for (int t = 0; t < 32; ++t) {
          const int r = 4 * t + (lane >> 4);
          bf16* const dst = row_ptr(t);
          if (row_base + r < M) *reinterpret_cast<u32x4*>(dst + c16 * 8) = d[t];
        }
      };
      if (plain_rows) {
        bf16* const p0 = cwave + (long long)(epi.rows.offset + row_base + (lane >> 4)) * ldc;
        store_rows([&](int t) { return p0 + (long long)(4 * t) * ldc; });
      } else {
        RowWalk w = row_walk(lane >> 4);
        store_rows([&](int) { bf16* const q = cwave + row_of(w) * ldc; row_step(w, 4); return q; });
      }
    } else {
      // fp32 staging in two 64-row halves (row r: 512 bytes, 16-byte chunk c at
      // c ^ (r & 15)); each half's residual rows are loaded first so their latency
      // overlaps the staging writes
      const int ch = lane & 31;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint2 res[32];
        auto load_rows = [&](auto row_ptr) {
#pragma unroll
          for (int t = 0; t < 32; ++t) {
            const int r = 64 * h + 2 * t + (lane >> 5);
            const bf16* const src = row_ptr(t);
            res[t] = make_uint2(0u, 0u);
            if (row_base + r < M) res[t] = *reinterpret_cast<const uint2*>(src + ch * 4);
          }
        };
        if (plain_rows) {
          bf16* const p0 = cwave + (long long)(epi.rows.offset + row_base + 64 * h + (lane >> 5)) * ldc;
          load_rows([&](int t) { return p0 + (long long)(2 * t) * ldc; });
        } else {
          RowWalk w = row_walk(64 * h + (lane >> 5));
          load_rows([&](int) { bf16* const q = cwave + row_of(w) * ldc; row_step(w, 2); return q; });
        }
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * h + ii;
          const int r = ii * 32 + fr;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                           acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
              const int cw = 8 * j + 2 * q + fk;
              *reinterpret_cast<float4*>(ep + r * 512 + ((cw ^ (r & 15)) << 4)) = v;
            }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        auto store_rows = [&](auto row_ptr) {
#pragma unroll
          for (int t = 0; t < 32; ++t) {
            const int r = 2 * t + (lane >> 5);
            const float4 f = *reinterpret_cast<const float4*>(ep + r * 512 + ((ch ^ (r & 15)) << 4));
            bf16* const dst = row_ptr(t);
            if (row_base + 64 * h + r < M) {
              const uint2 u = res[t];
              float v[4] = {__uint_as_float(u.x << 16) + f.x, __uint_as_float(u.x & 0xffff0000u) + f.y,
                            __uint_as_float(u.y << 16) + f.z, __uint_as_float(u.y & 0xffff0000u) + f.w};
              Store4<bf16>::store(dst + ch * 4, v);
            }
          }
        };
        if (plain_rows) {
          bf16* const p0 = cwave + (long long)(epi.rows.offset + row_base + 64 * h + (lane >> 5)) * ldc;
          store_rows([&](int t) { return p0 + (long long)(2 * t) * ldc; });
        } else {
          RowWalk w = row_walk(64 * h + (lane >> 5));
          store_rows([&](int) { bf16* const q = cwave + row_of(w) * ldc; row_step(w, 2); return q; });
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // this half's reads are done before the next overwrites it
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return;
  }
  Epilogue e_nb = epi;
  e_nb.bias = nullptr;   // already in the accumulators
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + i * 32 + fr;
    if (m >= M) continue;
    const long long row = epi.rows(m);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
        epilogue_row4<bf16, KIND>(e_nb, N, row, ncol + j * 32 + 8 * q, v);
      }
  }
}

// ------------------------------------------------------------------ fp32 kernel
// 64 x 64 tile, BK = 16, 256 threads with 4 x 4 outputs each (VALU FMA); used
// by fp32 models, where accuracy rather than throughput is the point.
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda,
                                                       const float* __restrict__ Bt, int ldb,
                                                       int M, int N, int K, Epilogue epi) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * FBM, n0 = blockIdx.x * FBN;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const float* pa = A + (long long)min(m0 + lrow, M - 1) * lda + lk;
  const float* pb = Bt + (long long)min(n0 + lrow, N - 1) * ldb + lk;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    const float4 va = *reinterpret_cast<const float4*>(pa + k0);
    const float4 vb = *reinterpret_cast<const float4*>(pb + k0);
    As[lk + 0][lrow] = va.x; As[lk + 1][lrow] = va.y; As[lk + 2][lrow] = va.z; As[lk + 3][lrow] = va.w;
    Bs[lk + 0][lrow] = vb.x; Bs[lk + 1][lrow] = vb.y; Bs[lk + 2][lrow] = vb.z; Bs[lk + 3][lrow] = vb.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; b[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m < M) epilogue_row4<float, KIND>(epi, N, epi.rows(m), n0 + tx * 4, acc[i]);
  }
}

int epi_kind(const Epilogue& e) { return e.residual ? kEpiResidual : (e.gelu ? kEpiGelu : kEpiPlain); }

}  // namespace

hipError_t gemm_init() { return hipSuccess; }

hipError_t launch_gemm_bf16(const bf16* A, int lda, const bf16* Bt, int ldb, int M, int N, int K,
                            const Epilogue& epi, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  switch (epi_kind(epi)) {
    case kEpiGelu:
      gemm_bf16_kernel<kEpiGelu><<<tiles, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi);
      break;
    case kEpiResidual:
      gemm_bf16_kernel<kEpiResidual><<<tiles, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi);
      break;
    default:
      gemm_bf16_kernel<kEpiPlain><<<tiles, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const float* A, int lda, const float* Bt, int ldb, int M, int N, int K,
                           const Epilogue& epi, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  dim3 grid((N + FBN - 1) / FBN, (M + FBM - 1) / FBM);
  switch (epi_kind(epi)) {
    case kEpiGelu:
      gemm_f32_kernel<kEpiGelu><<<grid, 256, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi);
      break;
    case kEpiResidual:
      gemm_f32_kernel<kEpiResidual><<<grid, 256, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi);
      break;
    default:
      gemm_f32_kernel<kEpiPlain><<<grid, 256, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi);
  }
  return hipGetLastError();
}

}  // namespace cem
