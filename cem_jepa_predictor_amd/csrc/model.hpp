// Host-side model: device weights, workspace, and the enqueue sequences of
// the predictor rollout and of the CEM plan step.
#pragma once

#include <map>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "cem_jepa.h"
#include "kernels.hpp"

namespace cem {

// Bytes of the per-device plan-state scratch behind cem_plan_noalloc.
constexpr size_t kPlanScratchBytes = size_t(8) << 20;

struct Status {
  cem_status code = CEM_OK;
  std::string msg;
  bool ok() const { return code == CEM_OK; }
  static Status Ok() { return {}; }
};
Status hip_status(hipError_t e, const char* what);

// RAII: make `device` current, restore the previous device on exit.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int device);
  ~DeviceGuard();
};

struct LayerW {
  float *ln1_g, *ln1_b, *b_qkv, *b_o, *ln2_g, *ln2_b, *b_1, *b_2;
  void *w_qkv_t, *w_o_t, *w_1_t, *w_2_t;   // transposed: [out, in]
  // fp8 models: w_qkv_t and w_1_t hold e4m3 codes scaled by 1 / ws_*, and b_qkv,
  // b_1 hold the biases divided by ws_* (what the fp8 GEMM epilogue expects)
  float ws_qkv = 1.f, ws_1 = 1.f;
  // LayerNorm-folded bf16 models: w_qkv_t and w_1_t hold bf16(diag(gamma) W) for the
  // LayerNorm before them, and b_qkv, b_1 hold [b + beta W | column sums of those bf16
  // values] (2 x out floats)
};

// Per-plan-shape device state: inputs copied in, per-round history out.
// Device state of the plan path, for `batch` independent problems planned together
// (one predictor batch of batch * n candidates).  Per round rd: samples
// x_hist[rd][b n + i][ha], energies e_hist[rd][b n + i], elites elites[rd][b][k];
// Gaussians mu_hist[rd][b][ha] (round 0 = the caller's); per problem z_obs,
// z_goal, s0 and the frame-0 tokens f0.
struct PlanState {
  int n = 0, k = 0, r = 0, h = 0, ha = 0, batch = 0;   // capacity
  void* mem = nullptr;
  float *x_hist = nullptr, *e_hist = nullptr, *mu_hist = nullptr, *sigma_hist = nullptr;
  int* elites = nullptr;
  float *zobs = nullptr, *zgoal = nullptr, *s0 = nullptr;
  void *zobs_t = nullptr, *f0 = nullptr;               // model dtype [batch, P, E], [batch, P, d]
  uint32_t* params = nullptr;
  int last_n = 0, last_k = 0, last_r = 0, last_h = 0, last_batch = 0;   // the last plan run
};

// n, k, rounds, horizon, clamp bits, batch
using GraphKey = std::tuple<int, int, int, int, uint32_t, uint32_t, int>;

}  // namespace cem

struct cem_model {
  cem_model_desc desc{};
  int device = 0;
  bool bf16 = false;     // bf16 activations and weights (also for fp8 models)
  bool fp8 = false;      // LayerNorm-fed projections with e4m3 operands
  bool ln_fold = false;  // bf16: LN1 / LN2 folded into the q|k|v and MLP-up GEMMs
  size_t esz = 4;        // bytes per weight / activation element
  int B = 0;             // tokens per frame block
  long long rows_max = 0;

  void* warena = nullptr;
  void* arena = nullptr;

  // weights
  void* w_in_t = nullptr;  // [d, E]
  float* b_in = nullptr;
  float *w_a = nullptr, *b_a = nullptr, *w_s = nullptr, *b_s = nullptr;  // fp32 [A|S, d], [d]
  std::vector<cem::LayerW> layers;
  float *lnf_g = nullptr, *lnf_b = nullptr, *b_out = nullptr;
  void* w_out_t = nullptr;  // [E, d]

  // workspace
  void *x = nullptr, *h = nullptr, *q = nullptr, *u = nullptr, *kv = nullptr, *zhat = nullptr,
       *f0 = nullptr, *zobs_t = nullptr;
  uint8_t* h8 = nullptr;   // fp8 models: e4m3 LayerNorm output [rows, d]
  float* hs = nullptr;     // and its row scales [rows]
  float* ln_stats = nullptr;   // LayerNorm-folded models: [rstd | mean] of the rows of one call
  float* ln_parts = nullptr;   // and, for d % 256 == 0, the residual GEMMs' per-64-column
                               // (mean, squared deviations) of the rows they write

  cem::PlanState plan;
  hipStream_t cap_stream = nullptr;
  std::map<cem::GraphKey, hipGraphExec_t> graphs;

  // kernel timers (dense GEMMs)
  bool timers = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  std::vector<double> ev_flop;
  size_t ev_used = 0;
};

namespace cem {

Status model_create(const cem_model_desc& d, const float* host_w, int device, cem_model** out);
void model_destroy(cem_model* m);

Status rollout(cem_model* m, const float* actions, int n, int horizon, const float* z_obs,
               const float* s0, void* z_pred, hipStream_t st);
// `batch` independent plan steps in one predictor batch; problem b uses plan id
// p.plan_id + b and the b-th slice of every per-problem argument.
Status plan(cem_model* m, const cem_params& p, int batch, const float* z_obs, const float* z_goal,
            const float* s0, float* mu, float* sigma, float* action, int32_t* best_idx,
            hipStream_t st);
// The single-problem plan with its plan state in the device's `scratch` array
// (kPlanScratchBytes): no allocation, kernels enqueued directly, the model's
// trace left untouched.
Status plan_noalloc(cem_model* m, const cem_params& p, const float* z_obs, const float* z_goal,
                    const float* s0, float* mu, float* sigma, float* action, int32_t* best_idx,
                    hipStream_t st);
Status plan_trace(cem_model* m, int kind, void* dst, size_t bytes, hipStream_t st);
Status timer_read(cem_model* m, int64_t* launches, double* ms, double* flop);

size_t weights_count(const cem_model_desc& d);
Status validate_desc(const cem_model_desc& d);

}  // namespace cem
