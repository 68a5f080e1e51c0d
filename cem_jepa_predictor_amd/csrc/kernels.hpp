// Host launchers of the gfx950 kernels.  Every launcher enqueues on `stream`
// and returns hipGetLastError() of its launch; shape checks happen in the
// callers (abi.cpp / model.cpp) before anything is enqueued.
#pragma once

#include "common.hpp"

namespace cem {

constexpr int kMaxBlocks = 8;   // frame blocks a query can attend (max horizon)

// --- sampler.hip ---------------------------------------------------------
// x[e] = clamp(mu[e % ha] + sigma[e % ha] * z[e], lo, hi), e < n * ha.
// dev_params (nullable): uint32 {seed_lo, seed_hi, plan_id, first_round} overriding
// the key and plan id and offsetting `round`, so a captured graph can be re-keyed
// (and a plan resumed) without re-capture.
// batch > 1: problem b samples with mu + b ha, sigma + b ha and plan id + b into
// x + b n ha (raw likewise), exactly as a batch-1 call with those arguments.
hipError_t launch_sample(const float* mu, const float* sigma, int n, int ha, uint64_t seed,
                         uint32_t round, uint32_t plan_id, const uint32_t* dev_params, float lo,
                         float hi, float* x, uint32_t* raw, hipStream_t stream, int batch = 1);
hipError_t launch_set_params(uint32_t* dev_params, uint64_t seed, uint32_t plan_id,
                             uint32_t first_round, hipStream_t stream);

// --- embed.hip -------------------------------------------------------------
template <typename T>
hipError_t launch_convert(const float* in, T* out, long long count, hipStream_t stream);
// Action and state token rows (rows n*B + 0 and n*B + 1 of x) for step t.
// Candidate n belongs to problem n / n_per, whose state is s0 + (n / n_per) S.
template <typename T>
hipError_t launch_embed_action_state(const float* X, int N, int H, int t, int A, int S,
                                     const float* s0, const float* wa, const float* ba,
                                     const float* ws, const float* bs, T* x, int B, int d,
                                     int n_per, hipStream_t stream);
// Frame rows n*B + 2 + p of x = f0[(n / n_per) P + p] for every candidate n.
template <typename T>
hipError_t launch_broadcast_frame(const T* f0, int P, int d, T* x, int N, int B, int n_per,
                                  hipStream_t stream);
// The rows of the first frame block that layer 0 needs once each, gathered from x
// [N*B, d] into xc [problems (B - 1) + N, d]: problem b's shared rows (rows 1 .. B-1 of
// its first candidate b n_per: the state token and the frame tokens) at b (B - 1) + j,
// then candidate k's action row (row k B) at problems (B - 1) + k.  N = problems n_per,
// d % 8 == 0.
hipError_t launch_gather_layer0(const bf16* x, int B, int d, int problems, int n_per, int N,
                                bf16* xc, hipStream_t stream);

// --- layernorm.hip -----------------------------------------------------------
// y[r] = (x[in_rows(r)] - mean) * rsqrt(var + eps) * g + b, fp32 statistics.
template <typename T>
hipError_t launch_layernorm(const T* x, int rows, int d, RowMap in_rows, const float* g,
                            const float* b, float eps, T* y, hipStream_t stream);
bool layernorm_supports(int d);
// fp8 output (d % 512 == 0): y8[r] = OCP e4m3 codes of LayerNorm(x[in_rows(r)]) scaled
// by 448 / (its largest magnitude), row_scale[r] = that magnitude / 448 (1 for a zero row).
hipError_t launch_layernorm_fp8(const bf16* x, int rows, int d, RowMap in_rows, const float* g,
                                const float* b, float eps, uint8_t* y8, float* row_scale,
                                hipStream_t stream);
// Row statistics of bf16 rows [rows, d] (d % 128 == 0): mean[r] and rstd[r] =
// 1 / sqrt(biased variance + eps), fp32, the LayerNorm kernel's arithmetic.
hipError_t launch_row_stats(const bf16* x, int rows, int d, float eps, float* mean, float* rstd,
                            hipStream_t stream);
// The same statistics of rows [rows, d] (d % 64 == 0) from the per-64-column partial
// statistics a residual GEMM wrote for them (Epilogue::stats).
hipError_t launch_row_stats_combine(const float* parts, int rows, int d, float eps, float* mean,
                                    float* rstd, hipStream_t stream);
// The same per-row quantization of fp32 rows [rows, cols] (cols % 8 == 0).
hipError_t launch_quantize_rows_fp8(const float* x, int rows, int cols, uint8_t* y8,
                                    float* row_scale, hipStream_t stream);

// --- gemm.hip ----------------------------------------------------------------
// out = epilogue(A[M, K] @ Bt[N, K]^T); N % 4 == 0; bf16 (MFMA): K % 64 == 0
// (hipErrorInvalidValue otherwise); fp32: K % 16 == 0.  epi.stats (bf16 residual
// kind only) also needs N % 256 == 0, one output (split >= N) with ld0 % 8 == 0 and
// a 16-byte aligned c0, identity rows and M < 2^28; the other launchers reject it.
hipError_t launch_gemm_bf16(const bf16* A, int lda, const bf16* Bt, int ldb, int M, int N,
                            int K, const Epilogue& epi, hipStream_t stream);
hipError_t launch_gemm_f32(const float* A, int lda, const float* Bt, int ldb, int M, int N,
                           int K, const Epilogue& epi, hipStream_t stream);
// bf16 with affine rows (a LayerNorm folded into the projection that follows it):
// out = epilogue(scale[m] ((A Bt^T)[m, n] - shift[m] col[n]) + bias[n]) with
// row_vals = [scale[M] | shift[M]] and epi.bias = [bias[N] | col[N]] (one array
// each, the second part right after the first); plain or GELU epilogue; K % 64 == 0.
hipError_t launch_gemm_bf16_rows(const bf16* A, int lda, const bf16* Bt, int ldb, int M, int N,
                                 int K, const float* row_vals, const Epilogue& epi,
                                 hipStream_t stream);
// fp8 operands (OCP e4m3 codes): out = epilogue(row_scale[m] * w_scale * (A Bt^T)[m, n]
// + bias[n]) with epi.bias holding bias / w_scale; plain or GELU epilogue only;
// K % 128 == 0 (hipErrorInvalidValue otherwise).
hipError_t launch_gemm_fp8(const uint8_t* A, int lda, const uint8_t* Bt, int ldb, int M, int N,
                           int K, const float* row_scale, float w_scale, const Epilogue& epi,
                           hipStream_t stream);
hipError_t gemm_init();   // caches the current device's CU count (persistent grid size)

// --- attention.hip -------------------------------------------------------------
// Queries: rows n*B + i of q (head h at columns h*dh); keys/values of frame
// block tau: rows n*B + j of kv[tau] (K at columns h*dh, V at d + h*dh).
// Every key of blocks 0..nblk-1 is visible to every query (block-causal mask
// with the queries in the last block).
struct AttnArgs {
  const void* q;
  const void* kv[kMaxBlocks];
  void* o;
  int ldq, ldkv, ldo;
  int n, heads, dh, d, B, nblk;
  float scale;
  // bf16, nblk == 1, optional: q, k and v of every row come from the compact q|k|v
  // block [c_problems (B - 1) + n, 3 d] of the gathered layer-0 rows (launch_gather_layer0
  // order): row 0 of candidate i at c_problems (B - 1) + i, row r >= 1 at
  // (i / c_n_per) (B - 1) + r - 1; q, kv and ldq / ldkv are then unused.
  const void* qkv_c;
  int c_problems, c_n_per;
};
hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t attention_init();   // one-time dynamic-LDS attribute
hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream);
bool attention_bf16_supports(int dh, int B);
bool attention_f32_supports(int dh);

// --- energy.hip ----------------------------------------------------------------
// E[i] = mean |zp[i] - g[(i / n_per) pe ...]| over pe elements.
template <typename T>
hipError_t launch_energy(const T* zp, const float* g, int n, long long pe, float* E, int n_per,
                         hipStream_t stream);

// --- select_refit.hip ---------------------------------------------------------------
// idx[k] = k smallest (E, index) pairs; if mu != nullptr also the elites'
// mean / population std over ha columns of X [n, ha].  batch > 1: problem b
// works on E + b n, X + b n ha into idx + b k, mu + b ha, sigma + b ha.
constexpr int kMaxSelect = 16384;
hipError_t launch_select_refit(const float* E, const float* X, int n, int k, int ha, int* idx,
                               float* mu, float* sigma, hipStream_t stream, int batch = 1);
// mu_next[t] = mu_prev[t + 1], sigma_next[t] = fmax(sigma_prev[t + 1], sigma_floor) for
// t < h - 1; step h - 1 = (mu_fill, sigma_fill).  h * a <= 1024; outputs may alias inputs.
hipError_t launch_warm_start(const float* mu_prev, const float* sigma_prev, int h, int a,
                             float mu_fill, float sigma_fill, float sigma_floor, float* mu_next,
                             float* sigma_next, hipStream_t stream);
hipError_t select_init();

}  // namespace cem
