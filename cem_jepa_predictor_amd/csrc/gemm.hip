// Dense projections of the predictor: out = epilogue(A[M, K] @ Bt[N, K]^T).
//
// Every linear layer of the action-conditioned predictor (fused q|k|v, output
// projection, MLP up with GELU, MLP down, frame in/out projections) goes
// through here.  These GEMMs carry about 95% of the plan step's FLOPs at the
// V-JEPA2-AC predictor shape (page "Real-Time Inference for JEPA World Model
// Architectures with Ray", section 01: ~8,000 predictor evaluations per
// action).  They are dense contractions for the matrix cores; with 256 x 256
// tiles what limits them on this part is the per-CU path that carries the
// operand slabs in and the results out (about 20 bytes per clock per CU for
// both together), which leaves the matrix cores busy about two thirds of the
// time.
//
// bf16 kernel (gfx950):
//  * 256 x 256 output tile per 512-thread workgroup: eight wave64s in a 2 x 4
//    grid, two per SIMD, each owning a 128 x 64 sub-tile = 4 x 2 tiles of
//    v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane).  With two
//    waves on a SIMD, one wave's MFMAs issue while the other waits on a load
//    or an LDS read; a single wave per SIMD spends most of a K-slab stalled
//    on its own memory instructions.
//  * The MFMA's first operand is the weight tile and its second the
//    activation tile, so each lane's accumulator quads hold 4 consecutive
//    output columns of one output row.
//  * Operands: global -> LDS directly (buffer_load_dwordx4 ... lds, no VGPR
//    staging) through a ring of five 32 KB entries, each holding one
//    operand's 256 x 64 slab (BK = 64): a slab takes two entries, so two and
//    a half slabs fit in LDS.  A K-slab of 64 makes every LDS row a whole
//    128-byte row piece of the operand, and the LDS-DMA path moves whole
//    128-byte pieces about 1.6x faster than the 64-byte halves of a 32-wide
//    slab.  128-byte LDS rows hold their eight 16-byte k-chunks at
//    c ^ ((r >> 1) & 7), so fragment reads are free of bank conflicts; each
//    lane loads the chunk that belongs at its slot.
//  * One barrier per K-slab, before its last substep (of four, 16 k-values
//    each): it publishes slab s+1 and frees slab s's two entries, which take
//    B of slab s+2 at once and A of slab s+2 one substep-0 later.  Every MFMA,
//    fragment read and load is placed explicitly (scheduling fences between
//    single instructions).
//  * Persistent: one workgroup per CU walks a sequence of tiles, and the
//    operand ring runs on across tile boundaries, so the next tile's first
//    slabs load while this tile's last slabs are computed and while its
//    results are stored; no tile pays a prologue.
//  * Tile order is XCD-aware: the dispatcher hands workgroup b to XCD b % 8;
//    each XCD owns a contiguous range of logical tiles, ordered in groups of
//    8 row-tiles (2 when a row of A holds 8 KB or more) to share A and B
//    panels in that XCD's L2, dealt round-robin to its workgroups.
//  * Ragged M / N: operand loads go through buffer resources bounded at the
//    tile's last valid row (the hardware returns zero beyond it).  Results, and
//    the residual rows the residual kind adds, go through buffer resources
//    bounded at row M as well (row-remapped outputs use masked stores).  With
//    only buffer operations in flight the compiler counts each wait on a
//    residual load exactly instead of draining every load.  K must be a
//    multiple of 64.
//  * Results leave through the ring entry that the tile's last slab frees
//    and that the next load into it waits for (4 KB a wave, 32 rows at a
//    time) as full 128-byte row pieces, stored non-temporally (this kernel
//    never reads them back).
//  * One kernel instantiation per epilogue kind (plain, GELU, residual), so
//    each carries only its own epilogue code.
//  * fp8 operands (OCP e4m3 codes, the gfx950 matrix cores' 8-bit format):
//    the same ring of 128-byte rows then holds 128 k-values per slab, each
//    slab is two substeps of v_mfma_f32_32x32x64_f8f6f4, and A fragments are
//    reloaded in place right after their last use (two fragment sets would not
//    fit the register budget of two waves per SIMD).  Row scales of A and one
//    scale for all of B are applied in the epilogue; the bias enters the
//    accumulators divided by both.  Plain and GELU epilogues.
//  * Affine rows (bf16): a LayerNorm folded into the projection after it, so
//    A is the raw residual stream and a per-row scale / shift and per-column
//    term are applied around the contraction (see the kernel's comment).
//  * Tile start: one MFMA per 32 x 32 block writes the bias (and the affine
//    row terms) into the accumulators from per-lane factors that were loaded
//    with bounds-checked buffer loads during the previous tile's first slab.
//
// Epilogue (fp32): + bias (already in the accumulators), optional GELU,
// optional residual add (the output already holds the residual stream),
// optional column split into two destinations (q -> Q buffer, k|v -> KV
// cache), optional output-row remap.  The residual kind can also write the
// statistics the next LayerNorm needs (its input is this output): for every
// 64-column piece of every row, the mean and sum of squared deviations of the
// rounded values, read back from the staging slots after the block's stores
// have been issued.
#include "kernels.hpp"

namespace cem {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS store that the compiler does not order against the operand loads in flight
// (it would wait for every outstanding buffer_load ... lds before any LDS store it
// cannot prove disjoint from them).  Used where the target region is known to be
// out of reach of every load in flight; the asm's memory clobber keeps later LDS
// reads behind it, and one wave's LDS accesses complete in order.
__device__ __forceinline__ void lds_write_b64(uint8_t* p, uint2 v) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_ptr_t)p;
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_write_b128(uint8_t* p, u32x4 v) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_ptr_t)p;
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
// A value every lane holds alike, moved to scalar registers: buffer resources built
// from it then stay scalar instead of being taken apart lane by lane.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

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
constexpr int BM = 256, BN = 256, BK = 64, NTHR = 512;
constexpr int BK8 = 128;                    // fp8 operands: k-values per 128-byte LDS row
constexpr int NE = 5;                       // entries in the operand ring
constexpr int ENT = BM * BK * 2;            // 32 KB: one operand slab (256 rows x 128 B)
// Row-tiles per tile group (the tiles of a group share A and B panels in one
// XCD's L2).  Measured on the isolated shapes at M = 206,400: K = 1024 runs best
// at 8 (MLP-up 1% slower at 2), K = 4096 (MLP-down) at 2 (3.5% faster than 8).
// Which CU computes which tile never changes a tile's arithmetic.
constexpr int GROUP_M = 8, GROUP_M_LONG_K = 2;


struct TileCoord {
  int m0, n0, rows_a, rows_b;   // rows_a = rows_b = 0: no tile (loads read zeros)
};

// A buffer resource over rows row0 .. row0 + rows - 1 of a row-major operand
// (ld elements of ES bytes), starting at column k: loads beyond it read zeros.
template <int ES>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, int row0, int rows,
                                                            int ld, int k) {
  const uint32_t bytes = ((uint32_t)rows * (uint32_t)ld - (uint32_t)k) * (uint32_t)ES;
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(base) + ((long long)row0 * ld + k) * ES),
      (short)0, (int)bytes, 0x00020000);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// AFF (affine rows): out = s_m ((A Bt^T)[m, n] - shift_m col_n) + w_scale bias_n with
// s_m = scale_m w_scale.  row_vals holds scale[M] and, when nrow == 2, shift[M] right
// after it; epi.bias holds bias[N] and, when ncol == 2, col[N] right after it (missing
// parts read as zero).  The accumulators start at bias_n / scale_m - shift_m col_n and
// the epilogue multiplies by s_m.
//  * F8 (implies AFF): operands are OCP fp8 e4m3 codes, A row m scaled by scale_m
//    and all of Bt by w_scale; epi.bias holds bias / w_scale.
//  * bf16 with AFF: a LayerNorm folded into the projection that follows it,
//    LN(x) W = rstd (x W' - mean 1^T W') + beta W with W' = diag(gamma) W:
//    scale = rstd, shift = mean, col = 1^T W', bias = b + beta W.
template <int KIND, bool F8, bool AFF>
__global__ __launch_bounds__(NTHR) void gemm_bf16_kernel(const void* __restrict__ A, int lda,
                                                         const void* __restrict__ Bt, int ldb,
                                                         int M, int N, int K, Epilogue epi,
                                                         const float* __restrict__ row_vals,
                                                         int nrow, float w_scale, int ncol) {
  static_assert(AFF || !F8, "fp8 operands always carry row scales");
  static_assert(!(AFF && KIND == kEpiResidual), "row scaling feeds the plain and GELU epilogues only");
  constexpr int ES = F8 ? 1 : 2;             // operand bytes per element
  constexpr int KS = F8 ? BK8 : BK;          // k-values per slab
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NE * ENT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN, tiles = tiles_m * tiles_n;
  const int KT = K / KS;

  // This workgroup's tiles.  The dispatcher hands workgroup b to XCD b % 8; XCD x
  // owns a contiguous range of logical tiles (groups of gm row-tiles sharing A and
  // B panels in that XCD's L2), dealt round-robin to its workgroups.
  const int gm = K * ES >= 8192 ? GROUP_M_LONG_K : GROUP_M;
  const int G = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int sx = (G >> 3) + (xcd < (G & 7) ? 1 : 0);
  const int tbase = tiles >> 3, trem = tiles & 7;
  const int tlo = xcd * tbase + min(xcd, trem), tcnt = tbase + (xcd < trem ? 1 : 0);
  auto coord = [&](int i) {
    TileCoord t{0, 0, 0, 0};
    const int idx = slot + i * sx;
    if (idx < tcnt) {
      const int L = tlo + idx;
      const int per_group = gm * tiles_n;
      const int g = L / per_group;
      const int first_m = g * gm;
      const int gsize = min(tiles_m - first_m, gm);
      const int in = L - g * per_group;
      t.m0 = (first_m + in % gsize) * BM;
      t.n0 = (in / gsize) * BN;
      t.rows_a = min(M - t.m0, BM);
      t.rows_b = min(N - t.n0, BN);
    }
    return t;
  };

  // Operand slabs: global -> LDS by buffer_load ... lds (16 bytes a lane; one
  // instruction fills 1 KB of LDS, lane l at byte 16 l).  The ring holds one
  // operand's 256 x 64 slab per 32 KB entry: A of sequence slab g in entry
  // 2g mod 5, B in 2g + 1 mod 5.  LDS row r (128 bytes, 8 chunks of 8 k-values)
  // holds logical chunk c at position c ^ ((r >> 1) & 7); each lane loads the
  // chunk that belongs at its slot, so one instruction reads 8 whole 128-byte
  // row pieces.  Wave w, instruction d: local rows 32 w + 8 d + lane / 8.
  const int dlrow = 32 * wave + (lane >> 3);
  const int dpos = lane & 7, dsw = (lane >> 4) & 3;
  const int dc0 = dpos ^ dsw, dc1 = dpos ^ (dsw | 4);           // d even / odd
  const int va0 = dlrow * lda * ES + (dc0 << 4), va1 = dlrow * lda * ES + (dc1 << 4);
  const int vb0 = dlrow * ldb * ES + (dc0 << 4), vb1 = dlrow * ldb * ES + (dc1 << 4);
  auto dma_a = [&](const TileCoord& t, int kt, int entry, int d) {
    const int kb = kt * KS;
    const __amdgpu_buffer_rsrc_t r = slab_rsrc<ES>(A, t.m0, t.rows_a, lda, t.rows_a ? kb : 0);
    const int v = ((d & 1) ? va1 : va0) + d * 8 * lda * ES;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds + entry * ENT + wave * 4096 + d * 1024), 16, v, 0, 0, 0);
  };
  auto dma_b = [&](const TileCoord& t, int kt, int entry, int d) {
    const int kb = kt * KS;
    const __amdgpu_buffer_rsrc_t r = slab_rsrc<ES>(Bt, t.n0, t.rows_b, ldb, t.rows_b ? kb : 0);
    const int v = ((d & 1) ? vb1 : vb0) + d * 8 * ldb * ES;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds + entry * ENT + wave * 4096 + d * 1024), 16, v, 0, 0, 0);
  };

  // 8 waves in a 2 x 4 grid, wave (wm, wn) owns output rows 128 wm .. +127 and
  // columns 64 wn .. +63: 4 x 2 tiles of v_mfma_f32_32x32x16_bf16.
  // Fragments: lane reads local row (l % 32) of a 32-row tile, k chunk 2 s + l / 32
  // of substep s (16 k-values each, four per slab).
  const int wm = wave >> 2, wn = wave & 3;
  const int fr = lane & 31, fk = lane >> 5;
  const int arow = (wm * 128 + fr) * 128;
  const int brow = (wn * 64 + fr) * 128;
  const int fsw = (fr >> 1) & 7;
  f32x16_t acc[4][2];
  bf16x8_t fa[2][4], fb[2][2];
  // fp8: v_mfma_f32_32x32x64_f8f6f4, lane l holding 32 k-values 32 (l / 32) ..
  // of its row: chunks 4 s + 2 (l / 32) and the next of substep s (two per slab).
  // A fragments are reloaded in place right after their last use; B has two sets.
  i32x8_t ga[4], gb[2][2];
  auto frag8 = [&](const uint8_t* p, int s) -> i32x8_t {
    const int c0 = 4 * s + 2 * fk;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p + ((c0 ^ fsw) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p + (((c0 + 1) ^ fsw) << 4));
    return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto frag8a = [&](int ea, int s, int i) { ga[i] = frag8(lds + ea * ENT + arow + i * 4096, s); };
  auto frag8b = [&](int ea, int s, int buf, int j) {
    const int eb = (ea + 1 == NE) ? 0 : ea + 1;
    gb[buf][j] = frag8(lds + eb * ENT + brow + j * 4096, s);
  };
  auto mfma8 = [&](int buf, int i, int j) {
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(gb[buf][j], ga[i], acc[i][j], 0, 0, 0, 0, 0, 0);
  };
  float rsc[4] = {1.f, 1.f, 1.f, 1.f};   // AFF: s_m of the lane's row in each 32-row block
  auto frag1 = [&](int ea, int s, int buf, int r) {
    const int pc = ((2 * s + fk) ^ fsw) << 4;
    if (r < 4) {
      fa[buf][r] = *reinterpret_cast<const bf16x8_t*>(lds + ea * ENT + arow + r * 4096 + pc);
    } else {
      const int eb = (ea + 1 == NE) ? 0 : ea + 1;
      fb[buf][r - 4] = *reinterpret_cast<const bf16x8_t*>(lds + eb * ENT + brow + (r - 4) * 4096 + pc);
    }
  };
  // The weight tile is the MFMA's first operand, so D[i][j] has j = output row
  // (lane % 32) and i = output column 8 (r / 4) + 4 (lane / 32) + r % 4.
  auto mfma1 = [&](int buf, int idx) {
    const int i = idx >> 1, j = idx & 1;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };
  // The accumulators start at A0[m, n] = bias_n / scale_m - shift_m col_n (bias_n
  // without AFF): a sum of two rank-1 terms, so one MFMA per 32 x 32 block writes it.
  // Lanes 0..31 bring the scale of row fr of each 32-row block and the bias of column
  // fr of each 32-column block, lanes 32..63 the shift and col.  Each fp32 factor is
  // split into three bf16 parts (v = v1 + v2 + v3, exact); k-slots 0..5 (lanes 0..31)
  // carry the six largest cross terms of (1 / scale)(bias), slots 8..13 (lanes 32..63)
  // those of (-shift)(col), leaving a relative error near 2^-24 per term.
  //
  // The factors come through bounds-checked buffer loads (out of range reads zero, so
  // a missing part costs nothing and needs no branch) into registers, issued for the
  // next tile during the current tile's first slab, just before its B loads: they land
  // as early as those instead of stalling the restart at the tile boundary.
  const __amdgpu_buffer_rsrc_t rrow = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(row_vals), (short)0, AFF && row_vals ? nrow * M * 4 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rcol = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(epi.bias), (short)0, epi.bias ? (AFF ? ncol : 1) * N * 4 : 0, 0x00020000);
  float nrv[4] = {1.f, 1.f, 1.f, 1.f}, ncv[2] = {0.f, 0.f};
  auto load_consts = [&](const TileCoord& t) {
    // lanes 32..63 read part 2 (shift, col); an exhausted grid reads out of range
    const int rbase = t.rows_a ? t.m0 + wm * 128 + fr + fk * M : 0x7fffffff / 4 - 256;
    const int cbase = t.rows_b ? t.n0 + wn * 64 + fr + fk * N : 0x7fffffff / 4 - 64;
    if constexpr (AFF) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = t.m0 + wm * 128 + 32 * i + fr;
        // rows past M read out of range (zero), also from part 2
        const int off = m < M ? (rbase + 32 * i) * 4 : 0x7ffffff0;
        nrv[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rrow, off, 0, 0));
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = t.n0 + wn * 64 + 32 * j + fr;
      const int off = n < N ? (cbase + 32 * j) * 4 : 0x7ffffff0;
      ncv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rcol, off, 0, 0));
    }
  };
  auto init_acc = [&]() {
    float sv[4], tv[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = fk == 0 ? 1.f : 0.f;
      if constexpr (AFF) {
        // rows past M read scale 0: their results are never stored
        sv[i] = fk == 0 ? __builtin_amdgcn_rcpf(nrv[i]) : -nrv[i];
        // every lane scales its rows in the epilogue: lanes 32..63 take lane - 32's
        rsc[i] = __shfl(nrv[i], fr, 64) * w_scale;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) tv[j] = ncv[j];
    auto split3 = [](float v, uint32_t& h1, uint32_t& h2, uint32_t& h3) {
      h1 = f32_to_bf16(v);
      const float r1 = v - __uint_as_float(h1 << 16);
      h2 = f32_to_bf16(r1);
      h3 = f32_to_bf16(r1 - __uint_as_float(h2 << 16));
    };
    bf16x8_t U[4], V[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h1, h2, h3;
      split3(sv[i], h1, h2, h3);
      // slots: s1 s1 s2 s1 s2 s3 0 0
      U[i] = __builtin_bit_cast(bf16x8_t, u32x4{h1 | (h1 << 16), h2 | (h1 << 16), h2 | (h3 << 16), 0u});
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t h1, h2, h3;
      split3(tv[j], h1, h2, h3);
      // slots: t1 t2 t1 t3 t2 t1 0 0
      V[j] = __builtin_bit_cast(bf16x8_t, u32x4{h1 | (h2 << 16), h1 | (h3 << 16), h2 | (h1 << 16), 0u});
    }
    const f32x16_t zero = {};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(V[j], U[i], zero, 0, 0, 0);
  };
#define CEM_WAIT(vm) __builtin_amdgcn_s_waitcnt(((vm) & 15) | (((vm) >> 4) << 14) | (0 << 8) | 0x0070)
#define F __builtin_amdgcn_sched_barrier(0)

  // tiles ahead: slab s + 2 is at most two tiles on (one-slab tiles)
  TileCoord T = coord(0), T1 = coord(1), T2 = coord(2);
  if (T.rows_a == 0) return;   // no tile for this workgroup (uniform)
  auto tile_at = [&](int off) -> TileCoord { return off == 0 ? T : (off == 1 ? T1 : T2); };
  load_consts(T);
  init_acc();
  F;
  // prologue: A and B of slabs 0 and 1 into entries 0..3
  {
    const int o1 = (KT == 1) ? 1 : 0, k1 = 1 - o1 * KT;
    const TileCoord t1 = tile_at(o1);
#pragma unroll
    for (int d = 0; d < 4; ++d) dma_a(T, 0, 0, d);
#pragma unroll
    for (int d = 0; d < 4; ++d) dma_b(T, 0, 1, d);
#pragma unroll
    for (int d = 0; d < 4; ++d) dma_a(t1, k1, 2, d);
#pragma unroll
    for (int d = 0; d < 4; ++d) dma_b(t1, k1, 3, d);
  }
  F;
  CEM_WAIT(8);   // slab 0 landed (this wave's part)
  __builtin_amdgcn_s_barrier();
  F;
  if constexpr (F8) {
#pragma unroll
    for (int j = 0; j < 2; ++j) frag8b(0, 0, 0, j);
#pragma unroll
    for (int i = 0; i < 4; ++i) frag8a(0, 0, i);
  } else {
#pragma unroll
    for (int r = 0; r < 6; ++r) frag1(0, 0, 0, r);
  }
  F;
  // The slab sequence runs on across tiles: slab KT + j is the next tile's slab j.
  // Slab s: substep 0 loads A of slab s + 2 into the entry that slab s - 1's B
  // left (after the epilogue when slab s - 1 ended a tile: the results are staged
  // there); substeps 0..2 read their successor's fragments; one barrier (slab
  // s + 1 landed everywhere, slab s's entries free); substep 3 reads slab s + 1's
  // first fragments and loads B of slab s + 2 into slab s's A entry.
  int ea = 0;                                   // entry of the current slab's A (B: ea + 1)
  int toff = (KT == 1) ? 2 : (KT == 2 ? 1 : 0);  // slab s + 2: tile offset and k-slab
  int tkt = 2 - toff * KT;
  for (int ti = 0;; ++ti) {
    int stage_ep = 0;
    for (int kt = 0; kt < KT; ++kt) {
      const int eb = (ea + 1 == NE) ? 0 : ea + 1;
      const int ea_n = (eb + 1 == NE) ? 0 : eb + 1;
      const int ea_p = (ea == 0) ? NE - 1 : ea - 1;   // slab s - 1's B entry
      const TileCoord Tt = tile_at(toff);
      if constexpr (F8) {
      // fp8 substep 0: B of substep 1 first, each A fragment reloaded after its last
      // use; A of slab s + 2
      mfma8(0, 0, 0); F; frag8b(ea, 1, 1, 0); F;
      mfma8(0, 0, 1); F; frag8b(ea, 1, 1, 1); F; frag8a(ea, 1, 0); F;
      mfma8(0, 1, 0); F; dma_a(Tt, tkt, ea_p, 0); F;
      mfma8(0, 1, 1); F; frag8a(ea, 1, 1); F; dma_a(Tt, tkt, ea_p, 1); F;
      mfma8(0, 2, 0); F; dma_a(Tt, tkt, ea_p, 2); F;
      mfma8(0, 2, 1); F; frag8a(ea, 1, 2); F; dma_a(Tt, tkt, ea_p, 3); F;
      mfma8(0, 3, 0); F;
      mfma8(0, 3, 1); F; frag8a(ea, 1, 3); F;
      // slab s + 1 landed (every load but the last 4: A of slab s + 2), own reads done
      CEM_WAIT(4);
      __builtin_amdgcn_s_barrier();
      F;
      // fp8 substep 1: slab s + 1's first fragments; B of slab s + 2
      mfma8(1, 0, 0); F; frag8b(ea_n, 0, 0, 0); F;
      mfma8(1, 0, 1); F; frag8b(ea_n, 0, 0, 1); F; frag8a(ea_n, 0, 0); F;
      if (kt == 0) load_consts(T1);
      F;
      mfma8(1, 1, 0); F; dma_b(Tt, tkt, ea, 0); F;
      mfma8(1, 1, 1); F; frag8a(ea_n, 0, 1); F; dma_b(Tt, tkt, ea, 1); F;
      mfma8(1, 2, 0); F; dma_b(Tt, tkt, ea, 2); F;
      mfma8(1, 2, 1); F; frag8a(ea_n, 0, 2); F; dma_b(Tt, tkt, ea, 3); F;
      mfma8(1, 3, 0); F;
      mfma8(1, 3, 1); F; frag8a(ea_n, 0, 3); F;
      } else {
      // substep 0
      mfma1(0, 0); F; frag1(ea, 1, 1, 0); F; frag1(ea, 1, 1, 1); F;
      mfma1(0, 1); F; frag1(ea, 1, 1, 2); F; frag1(ea, 1, 1, 3); F;
      mfma1(0, 2); F; frag1(ea, 1, 1, 4); F; frag1(ea, 1, 1, 5); F;
      mfma1(0, 3); F;
      dma_a(Tt, tkt, ea_p, 0); F;
      mfma1(0, 4); F;
      dma_a(Tt, tkt, ea_p, 1); F;
      mfma1(0, 5); F;
      dma_a(Tt, tkt, ea_p, 2); F;
      mfma1(0, 6); F;
      dma_a(Tt, tkt, ea_p, 3); F;
      mfma1(0, 7); F;
      // substep 1
      mfma1(1, 0); F; frag1(ea, 2, 0, 0); F; frag1(ea, 2, 0, 1); F;
      mfma1(1, 1); F; frag1(ea, 2, 0, 2); F; frag1(ea, 2, 0, 3); F;
      mfma1(1, 2); F; frag1(ea, 2, 0, 4); F; frag1(ea, 2, 0, 5); F;
      mfma1(1, 3); F; mfma1(1, 4); F; mfma1(1, 5); F; mfma1(1, 6); F; mfma1(1, 7); F;
      // substep 2
      mfma1(0, 0); F; frag1(ea, 3, 1, 0); F; frag1(ea, 3, 1, 1); F;
      mfma1(0, 1); F; frag1(ea, 3, 1, 2); F; frag1(ea, 3, 1, 3); F;
      mfma1(0, 2); F; frag1(ea, 3, 1, 4); F; frag1(ea, 3, 1, 5); F;
      mfma1(0, 3); F; mfma1(0, 4); F; mfma1(0, 5); F; mfma1(0, 6); F; mfma1(0, 7); F;
      // slab s + 1 landed (every load but the last 4: A of slab s + 2), own reads done
      CEM_WAIT(4);
      __builtin_amdgcn_s_barrier();
      F;
      // substep 3
      mfma1(1, 0); F; frag1(ea_n, 0, 0, 0); F; frag1(ea_n, 0, 0, 1); F;
      mfma1(1, 1); F; frag1(ea_n, 0, 0, 2); F; frag1(ea_n, 0, 0, 3); F;
      mfma1(1, 2); F; frag1(ea_n, 0, 0, 4); F; frag1(ea_n, 0, 0, 5); F;
      if (kt == 0) load_consts(T1);
      F;
      mfma1(1, 3); F;
      dma_b(Tt, tkt, ea, 0); F;
      mfma1(1, 4); F;
      dma_b(Tt, tkt, ea, 1); F;
      mfma1(1, 5); F;
      dma_b(Tt, tkt, ea, 2); F;
      mfma1(1, 6); F;
      dma_b(Tt, tkt, ea, 3); F;
      mfma1(1, 7); F;
      }
      if (++tkt == KT) { tkt = 0; ++toff; }
      stage_ep = eb;
      ea = ea_n;
    }

    const int ncol = T.n0 + wn * 64 + 4 * fk;
    const bool to_c0 = T.n0 + BN <= epi.split, to_c1 = T.n0 >= epi.split;
    bf16* const cbase = static_cast<bf16*>(to_c0 ? epi.c0 : epi.c1);
    const int ldc = to_c0 ? epi.ld0 : epi.ld1;
    const int cshift = to_c0 ? 0 : epi.split;
    if ((to_c0 || to_c1) && T.n0 + BN <= N && (ldc & 7) == 0 && (cshift & 7) == 0 &&
        (KIND == kEpiResidual ? epi.rows.group > M : epi.rows.group >= 8) &&
        ((uintptr_t)cbase & 15) == 0) {
      // Each wave stages its 128 x 64 result 32 rows at a time in its own 4 KB of
      // the free ring entry (row r: 128 bytes, 16-byte chunk c at c ^ ((r >> 1) & 7)),
      // then writes whole 128-byte row pieces (8 rows per store instruction).
      uint8_t* const ep = lds + stage_ep * ENT + wave * 4096;
      bf16* const cwave =
          reinterpret_cast<bf16*>(uniform_u64(reinterpret_cast<uintptr_t>(cbase + (T.n0 + wn * 64 - cshift))));
      const int ldcu = __builtin_amdgcn_readfirstlane(ldc);
      const int row_base = T.m0 + wm * 128;
      const bool plain_rows = epi.rows.group > M;
      // destination row of local row 8 t + lane / 8 of each 32-row block, walked in
      // steps of 8 (row map group >= 8)
      long long quot = 0;
      int rem = 0;
      if (!plain_rows) {
        const int m = row_base + (lane >> 3);
        quot = m / epi.rows.group;
        rem = m % epi.rows.group;
      }
      auto next_row = [&]() -> bf16* {
        bf16* q = cwave + (quot * epi.rows.stride + epi.rows.offset + rem) * ldc;
        rem += 8;
        if (rem >= epi.rows.group) { rem -= epi.rows.group; ++quot; }
        return q;
      };
      const int c16r = lane & 7;
      // Plain rows: one buffer resource per 8-row piece, its record count ending at
      // row M (rows past it read zero and are not written), and one per-lane byte
      // offset (row lane / 8, 16-byte chunk lane % 8).  The residual kind reads and
      // writes only through these, so every wait on its loads is counted exactly.
      const int vro = ((lane >> 3) * ldcu + c16r * 8) * 2;
      auto piece_rsrc = [&](int i, int t) {
        const int r0 = row_base + 32 * i + 8 * t;
        // rows of this piece inside M, clamped to 0..8 on the scalar unit (a clamp
        // written in C becomes a vector med3 and the resource a per-lane loop)
        int nr;
        asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, 8" : "=s"(nr) : "s"(M - r0) : "scc");
        bf16* const base = cwave + ((long long)epi.rows.offset + r0) * ldcu;
        return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, nr * ldcu * 2, 0x00020000);
      };
      if constexpr (KIND == kEpiResidual) {
        // output row statistics: pieces of 64 columns, one per wave, written as
        // (mean, sum of squared deviations) for rows below M
        const bool want_stats = epi.stats != nullptr;
        const __amdgpu_buffer_rsrc_t rstat = __builtin_amdgcn_make_buffer_rsrc(
            want_stats ? epi.stats + 2LL * ((T.n0 >> 6) + wn) * M : nullptr, (short)0, want_stats ? M * 8 : 0,
            0x00020000);
        // the residual rows, loaded two blocks ahead (16 bytes a lane, 8 rows per load)
        // into the registers the block before them has just left for the staging slots
        u32x4 res[2][4];
        auto load_res = [&](int i, u32x4 (&r)[4]) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            r[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(piece_rsrc(i, t), vro, 0, 0));
        };
        load_res(0, res[0]);
        load_res(1, res[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // residual rows into the staging slots
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int rr = 8 * t + (lane >> 3);
            lds_write_b128(ep + rr * 128 + ((c16r ^ ((rr >> 1) & 7)) << 4), res[i % 2][t]);
          }
          if (i + 2 < 4) load_res(i + 2, res[i % 2]);
          // add the accumulators in fp32 and round once, in place
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c16 = 4 * j + q;
              uint2* const slotp = reinterpret_cast<uint2*>(ep + fr * 128 + ((c16 ^ ((fr >> 1) & 7)) << 4) + fk * 8);
              const uint2 u = *slotp;
              uint2 o;
              o.x = pack_bf16x2(__uint_as_float(u.x << 16) + acc[i][j][4 * q],
                                __uint_as_float(u.x & 0xffff0000u) + acc[i][j][4 * q + 1]);
              o.y = pack_bf16x2(__uint_as_float(u.y << 16) + acc[i][j][4 * q + 2],
                                __uint_as_float(u.y & 0xffff0000u) + acc[i][j][4 * q + 3]);
              lds_write_b64(reinterpret_cast<uint8_t*>(slotp), o);
            }
          u32x4 d[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int rr = 8 * t + (lane >> 3);
            d[t] = *reinterpret_cast<const u32x4*>(ep + rr * 128 + ((c16r ^ ((rr >> 1) & 7)) << 4));
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) __builtin_amdgcn_raw_buffer_store_b128(d[t], piece_rsrc(i, t), vro, 0, 2);
          F;
          if (want_stats) {
            // row fr's 64 columns of this wave: 32 in this lane (read back from its
            // staging slots), 32 in lane fr + 32.  One pass in fp32 (bf16 pair products
            // are exact): the squared deviations are sum(v^2) - sum(v)^2 / 64, relative
            // error about 2^-17 (1 + mean^2 / variance) of the piece
            float s = 0.f, s2 = 0.f;
            const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
            for (int c16 = 0; c16 < 8; ++c16) {
              const uint2 o = *reinterpret_cast<const uint2*>(ep + fr * 128 + ((c16 ^ ((fr >> 1) & 7)) << 4) + fk * 8);
              const bf16x2_t px = __builtin_bit_cast(bf16x2_t, o.x), py = __builtin_bit_cast(bf16x2_t, o.y);
              s = __builtin_amdgcn_fdot2_f32_bf16(px, ones, s, false);
              s = __builtin_amdgcn_fdot2_f32_bf16(py, ones, s, false);
              s2 = __builtin_amdgcn_fdot2_f32_bf16(px, px, s2, false);
              s2 = __builtin_amdgcn_fdot2_f32_bf16(py, py, s2, false);
            }
            const auto sp = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
            const auto qp = __builtin_amdgcn_permlane32_swap(__float_as_uint(s2), __float_as_uint(s2), false, false);
            const float sum = __uint_as_float(sp[0]) + __uint_as_float(sp[1]);
            const float mean = sum * (1.0f / 64.0f);
            const float m2 = fmaxf(fmaf(-sum, mean, __uint_as_float(qp[0]) + __uint_as_float(qp[1])), 0.f);
            // lanes 0..31 write rows row_base + 32 i + fr; rows at or past M are out of range
            const int off = fk == 0 ? (row_base + 32 * i + fr) * 8 : 0x7ffffff0;
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(mean), __float_as_uint(m2)}, rstat, off, 0, 0);
          }
          F;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]};
              if constexpr (AFF) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= rsc[i];
              }
              if constexpr (KIND == kEpiGelu) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = gelu_bf16_path(v[e]);
              }
              uint2 u;
              u.x = pack_bf16x2(v[0], v[1]);
              u.y = pack_bf16x2(v[2], v[3]);
              const int c16 = 4 * j + q;
              lds_write_b64(ep + fr * 128 + ((c16 ^ ((fr >> 1) & 7)) << 4) + fk * 8, u);
            }
          u32x4 d[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int rr = 8 * t + (lane >> 3);
            d[t] = *reinterpret_cast<const u32x4*>(ep + rr * 128 + ((c16r ^ ((rr >> 1) & 7)) << 4));
          }
          if (plain_rows) {
#pragma unroll
            for (int t = 0; t < 4; ++t) __builtin_amdgcn_raw_buffer_store_b128(d[t], piece_rsrc(i, t), vro, 0, 2);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int m = row_base + i * 32 + 8 * t + (lane >> 3);
              bf16* const dst = next_row();
              if (m < M) __builtin_nontemporal_store(d[t], reinterpret_cast<u32x4*>(dst + c16r * 8));
            }
          }
          F;
        }
      }
    } else {
      Epilogue e_nb = epi;
      e_nb.bias = nullptr;   // already in the accumulators
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = T.m0 + wm * 128 + i * 32 + fr;
        if (m >= M) continue;
        const long long row = epi.rows(m);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]};
            if constexpr (AFF) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] *= rsc[i];
            }
            epilogue_row4<bf16, KIND>(e_nb, N, row, ncol + j * 32 + 8 * q, v);
          }
      }
    }
    // every wave has read its staged rows back: entry stage_ep takes the pending A load
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    F;
    if (T1.rows_a == 0) break;
    T = T1;
    T1 = T2;
    T2 = coord(ti + 3);
    --toff;
    init_acc();
    F;
  }
  CEM_WAIT(0);   // drain the dummy loads of the slabs past the last tile
#undef F
#undef CEM_WAIT
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

namespace {
constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices] = {};   // compute units per device, filled on first use

// Compute units of the current device (the persistent grid is one workgroup per CU).
hipError_t cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && g_cus[dev] > 0) {
    *cus = g_cus[dev];
    return hipSuccess;
  }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev] = *cus;
  return hipSuccess;
}
}  // namespace

hipError_t gemm_init() {
  int cus = 0;
  return cu_count(&cus);
}

hipError_t launch_gemm_bf16(const bf16* A, int lda, const bf16* Bt, int ldb, int M, int N, int K,
                            const Epilogue& epi, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % BK != 0) return hipErrorInvalidValue;
  // row statistics come from the staged epilogue, which every tile must take; their
  // buffer resources count bytes in 32 bits (8 per row)
  if (epi.stats && !(epi.residual && N % BN == 0 && epi.split >= N && (epi.ld0 & 7) == 0 &&
                     epi.rows.group > M && ((uintptr_t)epi.c0 & 15) == 0 && M < (1 << 28)))
    return hipErrorInvalidValue;
  int cus = 0;
  const hipError_t ce = cu_count(&cus);
  if (ce != hipSuccess) return ce;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int grid = tiles < cus ? tiles : cus;   // persistent: one workgroup per CU
  switch (epi_kind(epi)) {
    case kEpiGelu:
      gemm_bf16_kernel<kEpiGelu, false, false><<<grid, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi, nullptr, 0, 1.f, 1);
      break;
    case kEpiResidual:
      gemm_bf16_kernel<kEpiResidual, false, false><<<grid, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi, nullptr, 0, 1.f, 1);
      break;
    default:
      gemm_bf16_kernel<kEpiPlain, false, false><<<grid, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi, nullptr, 0, 1.f, 1);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_rows(const bf16* A, int lda, const bf16* Bt, int ldb, int M, int N, int K,
                                 const float* row_vals, const Epilogue& epi, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % BK != 0 || !row_vals || epi.residual || epi.stats) return hipErrorInvalidValue;
  int cus = 0;
  const hipError_t ce = cu_count(&cus);
  if (ce != hipSuccess) return ce;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int grid = tiles < cus ? tiles : cus;
  if (epi.gelu)
    gemm_bf16_kernel<kEpiGelu, false, true><<<grid, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi, row_vals, 2, 1.f, 2);
  else
    gemm_bf16_kernel<kEpiPlain, false, true><<<grid, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi, row_vals, 2, 1.f, 2);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t* A, int lda, const uint8_t* Bt, int ldb, int M, int N, int K,
                           const float* row_scale, float w_scale, const Epilogue& epi,
                           hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % BK8 != 0 || !row_scale || epi.residual || epi.stats) return hipErrorInvalidValue;
  int cus = 0;
  const hipError_t ce = cu_count(&cus);
  if (ce != hipSuccess) return ce;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int grid = tiles < cus ? tiles : cus;
  if (epi.gelu)
    gemm_bf16_kernel<kEpiGelu, true, true><<<grid, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi, row_scale, 1, w_scale, 1);
  else
    gemm_bf16_kernel<kEpiPlain, true, true><<<grid, NTHR, 0, stream>>>(A, lda, Bt, ldb, M, N, K, epi, row_scale, 1, w_scale, 1);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const float* A, int lda, const float* Bt, int ldb, int M, int N, int K,
                           const Epilogue& epi, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (epi.stats) return hipErrorInvalidValue;
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
