/*
 * cem_jepa.h - C ABI of the MI355X (gfx950) CEM plan step over an
 * action-conditioned, block-causal transformer predictor.
 *
 * Source of the method: page "Real-Time Inference for JEPA World Model
 * Architectures with Ray" (dev48.org).  Section 01, "Where the sixteen seconds
 * actually goes": one planning step encodes the camera frame and the goal once,
 * then runs rounds of the cross-entropy method (CEM): draw N candidate action
 * sequences from a Gaussian centred on the current best guess, push every one
 * through the predictor, score each result against the goal embedding, keep the
 * best K, re-centre the Gaussian on them; ten rounds; execute the first action.
 * Section 04 ("What we learned building it"): the observation and goal latents
 * stay resident for the whole plan, and per round only candidate actions go
 * out and energies come back.  Section 05: the predictor is frame-causal, so a
 * KV cache across rollout steps is exact.
 *
 * Conventions shared by every entry point
 *  - Pointers named "device" are device memory on the model's device (or, for
 *    the model-free calls, on the current device); the caller owns them, the
 *    library never frees them or keeps them past the call.
 *  - Host pointers (descriptors, host_weights) are read during the call only.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    All device work is enqueued asynchronously on it; a call returns once the
 *    work is enqueued.  One model serves one stream at a time.
 *  - Every call validates its arguments before enqueueing anything; on error
 *    it enqueues nothing and returns a negative cem_status, and
 *    cem_last_error() gives a thread-local message.  HIP runtime failures map
 *    to CEM_E_HIP.  No C++ exception crosses this boundary.
 *  - Layouts are row-major and dense; float is IEEE binary32; bf16 values are
 *    stored as uint16 (the upper half of the binary32 pattern).
 *  - Results are deterministic: identical inputs give bitwise-identical
 *    outputs, independent of how candidates are grouped into launches.
 */
#ifndef CEM_JEPA_H
#define CEM_JEPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CEM_OK = 0,
  CEM_E_ARG = -1,      /* null/misaligned pointer, bad enum, bad scalar */
  CEM_E_SHAPE = -2,    /* sizes inconsistent or beyond the model's maxima */
  CEM_E_DTYPE = -3,    /* element type not supported for this call */
  CEM_E_OOM = -4,      /* device allocation failed */
  CEM_E_HIP = -5,      /* a HIP runtime call failed */
  CEM_E_INTERNAL = -6
} cem_status;

/* Model / tensor element types.  CEM_FP8 (model dtype only): a bf16 model whose
 * two LayerNorm-fed projections (fused q|k|v and MLP up) run on OCP fp8 e4m3
 * operands (page section 06, "D. Model compression"; the 8-bit format of the
 * gfx950 matrix cores): their weights quantized with one scale per matrix at
 * create time, the LayerNorm outputs quantized per token row, fp32
 * accumulation, both scales applied to the result; activations, every other
 * projection, attention and the rollout output stay bf16.  Needs d_model % 512
 * == 0. */
typedef enum { CEM_F32 = 0, CEM_BF16 = 1, CEM_FP8 = 2 } cem_dtype;

/* Predictor shape.  Frame block = 1 action token + 1 state token + `patches`
 * frame tokens (B = patches + 2).  `max_samples` and `max_horizon` size the
 * workspace allocated at create time.  Limits (cem_model_create and
 * cem_weights_count return CEM_E_SHAPE otherwise):
 *  - d_model one of 128, 256, 384, 512, 768, 1024, 1536, 2048, 4096, and a
 *    multiple of heads;
 *  - head dim d_model / heads: exactly 64 for CEM_BF16 and CEM_FP8 models;
 *    16, 32, 64 or 128 for CEM_F32 models;
 *  - CEM_BF16 / CEM_FP8: patches + 2 <= 320 (one frame block's keys fit the
 *    attention kernel's LDS); CEM_FP8 also needs d_model % 512 == 0;
 *  - d_mlp and enc_dim multiples of 64 in [64, 65536]; patches in [1, 4096];
 *  - layers in [1, 256]; action_dim and state_dim in [1, 32], equal when
 *    max_horizon > 1 (the state advances by the action);
 *  - max_horizon in [1, 8]; max_samples in [1, 16384]; ln_eps > 0, finite;
 *  - max_samples * (patches + 2) <= 2^30 rows. */
typedef struct {
  int32_t layers, d_model, heads, d_mlp, patches, enc_dim;
  int32_t action_dim, state_dim, max_horizon, max_samples;
  int32_t dtype;   /* cem_dtype: CEM_F32 = fp32 everywhere; CEM_BF16 = bf16
                      weights and activations, fp32 accumulation, LayerNorm
                      statistics, softmax and energies; the LayerNorm before
                      q|k|v and before the MLP is folded into those projections
                      (gain into the weights, shift into the bias, row mean and
                      rstd applied around the contraction) */
  float ln_eps;
} cem_model_desc;

/* CEM settings (page section 01: 800 candidates, best 80, ten rounds). */
typedef struct {
  int32_t n_samples;   /* N, 1..max_samples */
  int32_t n_elites;    /* K, 1..N */
  int32_t rounds;      /* R >= 1 */
  int32_t horizon;     /* H, 1..max_horizon */
  float clamp_lo, clamp_hi;   /* sampled actions are clamped to [lo, hi] */
  uint64_t seed;       /* Philox key */
  uint32_t plan_id;    /* Philox counter word 2: distinct plans, distinct draws */
  int32_t use_graph;   /* 1: capture the R rounds once per shape as a HIP graph
                          and replay it; 0: enqueue kernels directly */
  uint32_t first_round;   /* Philox counter word 1 of the first round (round r of
                             this call draws with first_round + r): 0 for a fresh
                             plan; r0 resumes a plan after r0 rounds from the mu and
                             sigma it returned, drawing exactly what an uninterrupted
                             plan draws in its rounds r0, r0 + 1, ... */
} cem_params;

typedef struct cem_model cem_model;   /* opaque: device weights + workspace */

/* Thread-local text of the last non-OK status (never NULL). */
const char* cem_last_error(void);

/* Number of floats in the flat weight buffer for `desc`.  Canonical order
 * (matrices stored [in, out], so a layer computes x @ W + b):
 *   w_in[E,d] b_in[d] w_a[A,d] b_a[d] w_s[S,d] b_s[d]
 *   per layer: ln1_g[d] ln1_b[d] w_qkv[d,3d] b_qkv[3d] w_o[d,d] b_o[d]
 *              ln2_g[d] ln2_b[d] w_1[d,F] b_1[F] w_2[F,d] b_2[d]
 *   lnf_g[d] lnf_b[d] w_out[d,E] b_out[E]
 * w_qkv's columns are [q | k | v]; head h owns columns h*dh..h*dh+dh-1 of each. */
cem_status cem_weights_count(const cem_model_desc* desc, size_t* n_floats);

/* Create a model on `device`: converts the host fp32 weights to the model
 * dtype (round to nearest even for bf16; for CEM_BF16 the LayerNorm gains are
 * multiplied into the following weights before rounding), lays them out for the kernels,
 * uploads them and allocates the workspace for max_samples x max_horizon
 * (including the KV cache).  Synchronous.  *out receives the handle. */
cem_status cem_model_create(const cem_model_desc* desc, const float* host_weights,
                            size_t n_floats, int32_t device, cem_model** out);
cem_status cem_model_destroy(cem_model* model);

/* One full CEM plan step (page section 01).
 *   z_obs, z_goal : device fp32 [P, E]  observation / goal embeddings
 *   s0            : device fp32 [S]     current state
 *   mu, sigma     : device fp32 [H, A]  in: initial Gaussian; out: final refit
 *   action        : device fp32 [A]     out: mu_R[0, :], the action to execute
 *   best_idx      : device int32 [1]    out: best candidate of the last round
 *                                        (nullable)
 * Round r samples X_r = clamp(mu_r + sigma_r * z, lo, hi) with Philox-4x32-10
 * (counter (e >> 2, r, plan_id, 0), key = seed) and float64 Box-Muller, rolls
 * every candidate through the predictor (autoregressive over H frame blocks,
 * block-causal, KV cache), scores E[n] = mean |z_H[n] - z_goal|, keeps the K
 * lowest (energy, index) pairs (NaN ranks as +inf) and refits mu, sigma as the
 * elites' mean and population std (float64 accumulation).  The per-round
 * samples, energies, elites and Gaussians stay on the device for
 * cem_plan_trace until the next cem_plan on this model. */
cem_status cem_plan(cem_model* model, const cem_params* params, const float* z_obs,
                    const float* z_goal, const float* s0, float* mu, float* sigma,
                    float* action, int32_t* best_idx, void* stream);

/* Fleet batching (page section 06, "C. Fleet-level batching"): `batch`
 * independent plan steps -- e.g. one per robot -- searched together, their
 * candidates packed into one predictor batch per round.  Problem b plans with
 * plan id params->plan_id + b on its own slice of every per-problem argument:
 *   z_obs, z_goal : device fp32 [batch, P, E];  s0 : device fp32 [batch, S]
 *   mu, sigma     : device fp32 [batch, H, A]   in/out as in cem_plan
 *   action        : device fp32 [batch, A];  best_idx : device int32 [batch]
 * params->n_samples and n_elites are per problem (batch * n_samples <=
 * max_samples, batch <= 4096).  Problem b's results equal those of cem_plan
 * with plan id params->plan_id + b on its own inputs, bit for bit.  The trace
 * of a batched plan holds every problem: actions [R, batch * N, H, A], energies
 * [R, batch * N], elites [R, batch, K] (indices within each problem), mu and
 * sigma [R + 1, batch, H, A]. */
cem_status cem_plan_batched(cem_model* model, const cem_params* params, int32_t batch,
                            const float* z_obs, const float* z_goal, const float* s0, float* mu,
                            float* sigma, float* action, int32_t* best_idx, void* stream);

/* cem_plan without allocation, for callers that cannot call hipMalloc: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments, results and errors are those of cem_plan, and the results are
 * bitwise equal to cem_plan's for the same arguments.  Differences:
 *  - The plan state (per-round samples, energies, elites and Gaussians, the
 *    staged z_obs / z_goal / s0 and the frame-0 tokens) lives in a static device
 *    array of 8 MiB (8388608 bytes) that the library holds on each device it runs
 *    on until the process ends.  Bytes needed, each term rounded up to 256:
 *    R N H A 4 + R N 4 + 2 (R + 1) H A 4 + R K 4 + 2 P E 4 + 256 + P E es + P d es
 *    + 16, with es = 4 for CEM_F32 and 2 otherwise (the 800 x 10 plan at the
 *    V-JEPA2-AC shape needs about 4.4 MB).  A plan that needs more returns
 *    CEM_E_SHAPE and enqueues nothing.
 *  - Every call on a device shares that device's array: calls that overlap on
 *    one GPU (two streams, or two models on one device) race and corrupt each
 *    other.  The array keeps the last call's contents; nothing in it needs to
 *    start at zero.
 *  - Kernels and copies are enqueued directly on `stream` (params->use_graph is
 *    ignored), so a caller may capture them into its own graph.  The model's
 *    workspace (allocated by cem_model_create) is used as by cem_plan.
 *  - cem_plan_trace keeps describing the last cem_plan, not this call.
 *  - Kernel timers must be off on the model (CEM_E_ARG otherwise). */
cem_status cem_plan_noalloc(cem_model* model, const cem_params* params, const float* z_obs,
                            const float* z_goal, const float* s0, float* mu, float* sigma,
                            float* action, int32_t* best_idx, void* stream);

typedef enum {
  CEM_TRACE_ACTIONS = 0,  /* fp32 [R, N, H, A] sampled candidates */
  CEM_TRACE_ENERGY = 1,   /* fp32 [R, N] energies */
  CEM_TRACE_ELITES = 2,   /* int32 [R, K] elite indices, ascending (energy, index) */
  CEM_TRACE_MU = 3,       /* fp32 [R + 1, H, A] Gaussian means, mu_0 first */
  CEM_TRACE_SIGMA = 4     /* fp32 [R + 1, H, A] Gaussian std devs */
} cem_trace_kind;

/* Copy part of the last plan's trace into device memory `dst` of `bytes`
 * bytes (must equal the size above for that plan).  Asynchronous on stream. */
cem_status cem_plan_trace(cem_model* model, int32_t kind, void* dst, size_t bytes,
                          void* stream);

/* Predictor rollout alone (page section 01, "pushes every one through the
 * predictor"; section 05, KV cache across rollout steps).
 *   actions : device fp32 [n, horizon, A]
 *   z_obs   : device fp32 [P, E];  s0 : device fp32 [S]
 *   z_pred  : device [n, P, E] in the model dtype: the last predicted frame */
cem_status predictor_rollout(cem_model* model, const float* actions, int32_t n,
                             int32_t horizon, const float* z_obs, const float* s0,
                             void* z_pred, void* stream);

/* L1 energy (page section 01, "scores the results against the goal"):
 *   energy[i] = (1 / (p * e)) * sum_{j < p*e} |z_pred[i, j] - z_goal[j]|
 * z_pred device [n, p, e] of `dtype` (fp32 or bf16), z_goal device fp32
 * [p, e], energy device fp32 [n].  Accumulates in fp32 in a fixed order. */
cem_status energy_l1(const void* z_pred, int32_t dtype, const float* z_goal, int32_t n,
                     int32_t p, int32_t e, float* energy, void* stream);

/* Elite selection and refit (page section 01, "keeps the best 80, and
 * re-centers the Gaussian on them"):
 *   energy    : device fp32 [n];  actions : device fp32 [n, h, a]
 *   elite_idx : device int32 [k] out, ascending by (energy, index), NaN = +inf
 *   mu, sigma : device fp32 [h, a] out, mean and population std of the elites
 * n <= 16384, k <= n. */
cem_status elite_refit(const float* energy, const float* actions, int32_t n, int32_t k,
                       int32_t h, int32_t a, int32_t* elite_idx, float* mu, float* sigma,
                       void* stream);

/* Warm start of the next control step (page section 06, "B. Warm-started
 * CEM"): receding-horizon control executes only the plan's first action; the
 * rest of the plan seeds the next step's Gaussian, one step earlier, instead of
 * a fresh one, so the next plan can converge in fewer rounds.
 *   mu_prev, sigma_prev : device fp32 [h, a]  a plan's final mu, sigma
 *   mu_next, sigma_next : device fp32 [h, a]  out (may alias the inputs)
 * For t < h - 1: mu_next[t] = mu_prev[t + 1] and sigma_next[t] =
 * fmax(sigma_prev[t + 1], sigma_floor) (a NaN width becomes sigma_floor); the
 * last step starts fresh: mu_next[h - 1] = mu_fill, sigma_next[h - 1] =
 * sigma_fill.  h = 1 is a plain reset.  sigma_floor = sigma_fill resets every
 * width to at least the fresh one; 0 keeps the previous widths.
 * h * a <= 1024; mu_fill, sigma_fill, sigma_floor finite, sigma_fill > 0,
 * sigma_floor >= 0.  Pass the result as cem_plan's mu, sigma. */
cem_status cem_warm_start(const float* mu_prev, const float* sigma_prev, int32_t h, int32_t a,
                          float mu_fill, float sigma_fill, float sigma_floor, float* mu_next,
                          float* sigma_next, void* stream);

/* Sampler alone: actions[n, h, a] = clamp(mu + sigma * z, lo, hi) for round
 * `round` (see cem_plan); raw_words (nullable) receives each element's Philox
 * word, uint32 [n * h * a]. */
cem_status cem_sample(const float* mu, const float* sigma, int32_t n, int32_t h, int32_t a,
                      uint64_t seed, uint32_t round, uint32_t plan_id, float lo, float hi,
                      float* actions, uint32_t* raw_words, void* stream);

/* fp8 row quantization alone (the step that feeds CEM_FP8 projections): for each
 * row r of x (device fp32 [rows, cols], cols % 8 == 0), scale[r] = amax_r / 448
 * (1 for an all-zero row) and codes[r, c] = e4m3(clamp(x[r, c] * (448 / amax_r),
 * -448, 448)), rounded to nearest even; codes device uint8 [rows, cols], scale
 * device fp32 [rows]. */
cem_status cem_fp8_quantize_rows(const float* x, int32_t rows, int32_t cols, uint8_t* codes,
                                 float* scale, void* stream);

/* Top-K alone: idx[k] = the k smallest (energy, index) pairs, ascending. */
cem_status topk_select(const float* energy, int32_t n, int32_t k, int32_t* idx, void* stream);

/* Kernel timers for measurement.  When enabled, cem_plan and
 * predictor_rollout enqueue directly (no graph) and bracket every launch of
 * the predictor's dense GEMMs with HIP events on the launch stream.
 * cem_timer_read waits for those events, returns the number of launches and
 * their summed duration and useful FLOPs since the last read, and resets. */
cem_status cem_timer_enable(cem_model* model, int32_t enable);
cem_status cem_timer_read(cem_model* model, int64_t* launches, double* total_ms,
                          double* total_flop);

#ifdef __cplusplus
}
#endif
#endif /* CEM_JEPA_H */
