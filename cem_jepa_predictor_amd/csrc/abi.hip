// extern "C" boundary: argument validation, status codes, thread-local error
// text.  Nothing is enqueued unless every argument checks out; no C++
// exception crosses this boundary.
#include <hip/hip_runtime.h>

#include <cmath>
#include <new>
#include <string>

#include "cem_jepa.h"
#include "model.hpp"

namespace {

thread_local std::string g_last_error = "no error";

cem_status fail(cem_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
cem_status finish(const cem::Status& s) {
  if (s.ok()) return CEM_OK;
  return fail(s.code, s.msg);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <typename F>
cem_status guarded(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return fail(CEM_E_OOM, "host allocation failed");
  } catch (const std::exception& e) {
    return fail(CEM_E_INTERNAL, e.what());
  } catch (...) {
    return fail(CEM_E_INTERNAL, "unknown internal error");
  }
}

// selection needs a one-time LDS attribute on each device the model-free calls run on
cem_status ensure_select_ready() {
  static thread_local int ready_mask = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CEM_E_HIP, "hipGetDevice failed");
  if (dev < 31 && (ready_mask & (1 << dev))) return CEM_OK;
  const hipError_t e = cem::select_init();
  if (e != hipSuccess) return fail(CEM_E_HIP, std::string("select_init: ") + hipGetErrorString(e));
  if (dev < 31) ready_mask |= 1 << dev;
  return CEM_OK;
}

cem_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return CEM_OK;
  return fail(e == hipErrorOutOfMemory ? CEM_E_OOM : CEM_E_HIP,
              std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

namespace {
cem_status plan_checked(cem_model* model, const cem_params* p, int32_t batch, const float* z_obs,
                        const float* z_goal, const float* s0, float* mu, float* sigma, float* action,
                        int32_t* best_idx, void* stream, bool noalloc = false) {
  if (!model || !p || !z_obs || !z_goal || !s0 || !mu || !sigma || !action)
    return fail(CEM_E_ARG, "null argument");
  if (!aligned(z_obs, 4) || !aligned(z_goal, 4) || !aligned(s0, 4) || !aligned(mu, 4) ||
      !aligned(sigma, 4) || !aligned(action, 4) || (best_idx && !aligned(best_idx, 4)))
    return fail(CEM_E_ARG, "misaligned pointer (4-byte alignment required)");
  const cem_model_desc& d = model->desc;
  if (batch < 1 || batch > 4096) return fail(CEM_E_SHAPE, "batch must be in [1, 4096]");
  if (p->n_samples < 1 || (long long)p->n_samples * batch > d.max_samples)
    return fail(CEM_E_SHAPE, "n_samples must be >= 1 with batch * n_samples <= max_samples");
  if (p->n_elites < 1 || p->n_elites > p->n_samples)
    return fail(CEM_E_SHAPE, "n_elites must be in [1, n_samples]");
  if (p->rounds < 1 || p->rounds > 4096) return fail(CEM_E_SHAPE, "rounds must be in [1, 4096]");
  if (p->horizon < 1 || p->horizon > d.max_horizon)
    return fail(CEM_E_SHAPE, "horizon must be in [1, max_horizon]");
  if (!std::isfinite(p->clamp_lo) || !std::isfinite(p->clamp_hi) || p->clamp_lo > p->clamp_hi)
    return fail(CEM_E_ARG, "clamp bounds must be finite with lo <= hi");
  if (p->use_graph != 0 && p->use_graph != 1) return fail(CEM_E_ARG, "use_graph must be 0 or 1");
  if ((uint64_t)p->plan_id + (uint64_t)(batch - 1) > 0xffffffffull)
    return fail(CEM_E_ARG, "plan_id + batch - 1 must fit in 32 bits");
  if (noalloc)
    return finish(cem::plan_noalloc(model, *p, z_obs, z_goal, s0, mu, sigma, action, best_idx,
                                    static_cast<hipStream_t>(stream)));
  return finish(cem::plan(model, *p, batch, z_obs, z_goal, s0, mu, sigma, action, best_idx,
                          static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" {

const char* cem_last_error(void) { return g_last_error.c_str(); }

cem_status cem_weights_count(const cem_model_desc* desc, size_t* n_floats) {
  return guarded([&]() -> cem_status {
    if (!desc || !n_floats) return fail(CEM_E_ARG, "null argument");
    const cem::Status v = cem::validate_desc(*desc);
    if (!v.ok()) return finish(v);
    *n_floats = cem::weights_count(*desc);
    return CEM_OK;
  });
}

cem_status cem_model_create(const cem_model_desc* desc, const float* host_weights, size_t n_floats,
                            int32_t device, cem_model** out) {
  return guarded([&]() -> cem_status {
    if (!desc || !host_weights || !out) return fail(CEM_E_ARG, "null argument");
    *out = nullptr;
    const cem::Status v = cem::validate_desc(*desc);
    if (!v.ok()) return finish(v);
    const size_t want = cem::weights_count(*desc);
    if (n_floats != want)
      return fail(CEM_E_SHAPE, "weight count " + std::to_string(n_floats) + " != expected " +
                                   std::to_string(want));
    for (size_t i = 0; i < n_floats; ++i)
      if (!std::isfinite(host_weights[i])) return fail(CEM_E_ARG, "non-finite weight at index " + std::to_string(i));
    return finish(cem::model_create(*desc, host_weights, device, out));
  });
}

cem_status cem_model_destroy(cem_model* model) {
  return guarded([&]() -> cem_status {
    if (!model) return fail(CEM_E_ARG, "null model");
    cem::model_destroy(model);
    return CEM_OK;
  });
}


cem_status cem_plan(cem_model* model, const cem_params* p, const float* z_obs, const float* z_goal,
                    const float* s0, float* mu, float* sigma, float* action, int32_t* best_idx,
                    void* stream) {
  return guarded([&]() -> cem_status {
    return plan_checked(model, p, 1, z_obs, z_goal, s0, mu, sigma, action, best_idx, stream);
  });
}

cem_status cem_plan_batched(cem_model* model, const cem_params* p, int32_t batch, const float* z_obs,
                            const float* z_goal, const float* s0, float* mu, float* sigma,
                            float* action, int32_t* best_idx, void* stream) {
  return guarded([&]() -> cem_status {
    return plan_checked(model, p, batch, z_obs, z_goal, s0, mu, sigma, action, best_idx, stream);
  });
}

cem_status cem_plan_noalloc(cem_model* model, const cem_params* p, const float* z_obs,
                            const float* z_goal, const float* s0, float* mu, float* sigma,
                            float* action, int32_t* best_idx, void* stream) {
  return guarded([&]() -> cem_status {
    return plan_checked(model, p, 1, z_obs, z_goal, s0, mu, sigma, action, best_idx, stream, true);
  });
}

cem_status cem_plan_trace(cem_model* model, int32_t kind, void* dst, size_t bytes, void* stream) {
  return guarded([&]() -> cem_status {
    if (!model || !dst) return fail(CEM_E_ARG, "null argument");
    if (!aligned(dst, 4)) return fail(CEM_E_ARG, "misaligned pointer");
    return finish(cem::plan_trace(model, kind, dst, bytes, static_cast<hipStream_t>(stream)));
  });
}

cem_status predictor_rollout(cem_model* model, const float* actions, int32_t n, int32_t horizon,
                             const float* z_obs, const float* s0, void* z_pred, void* stream) {
  return guarded([&]() -> cem_status {
    if (!model || !actions || !z_obs || !s0 || !z_pred) return fail(CEM_E_ARG, "null argument");
    if (!aligned(actions, 4) || !aligned(z_obs, 4) || !aligned(s0, 4) || !aligned(z_pred, 4))
      return fail(CEM_E_ARG, "misaligned pointer (4-byte alignment required)");
    if (n < 1 || n > model->desc.max_samples) return fail(CEM_E_SHAPE, "n must be in [1, max_samples]");
    if (horizon < 1 || horizon > model->desc.max_horizon)
      return fail(CEM_E_SHAPE, "horizon must be in [1, max_horizon]");
    return finish(cem::rollout(model, actions, n, horizon, z_obs, s0, z_pred,
                               static_cast<hipStream_t>(stream)));
  });
}

cem_status energy_l1(const void* z_pred, int32_t dtype, const float* z_goal, int32_t n, int32_t p,
                     int32_t e, float* energy, void* stream) {
  return guarded([&]() -> cem_status {
    if (!z_pred || !z_goal || !energy) return fail(CEM_E_ARG, "null argument");
    if (dtype != CEM_F32 && dtype != CEM_BF16) return fail(CEM_E_DTYPE, "dtype must be CEM_F32 or CEM_BF16");
    if (n < 0 || p < 1 || e < 1) return fail(CEM_E_SHAPE, "need n >= 0, p >= 1, e >= 1");
    if (!aligned(z_pred, dtype == CEM_BF16 ? 2 : 4) || !aligned(z_goal, 4) || !aligned(energy, 4))
      return fail(CEM_E_ARG, "misaligned pointer");
    const long long pe = (long long)p * e;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t r =
        dtype == CEM_BF16 ? cem::launch_energy<cem::bf16>(static_cast<const cem::bf16*>(z_pred), z_goal, n, pe, energy, n, st)
                          : cem::launch_energy<float>(static_cast<const float*>(z_pred), z_goal, n, pe, energy, n, st);
    return check_hip(r, "energy kernel");
  });
}

cem_status elite_refit(const float* energy, const float* actions, int32_t n, int32_t k, int32_t h,
                       int32_t a, int32_t* elite_idx, float* mu, float* sigma, void* stream) {
  return guarded([&]() -> cem_status {
    if (!energy || !actions || !elite_idx || !mu || !sigma) return fail(CEM_E_ARG, "null argument");
    if (!aligned(energy, 4) || !aligned(actions, 4) || !aligned(elite_idx, 4) || !aligned(mu, 4) ||
        !aligned(sigma, 4))
      return fail(CEM_E_ARG, "misaligned pointer");
    if (n < 1 || n > cem::kMaxSelect) return fail(CEM_E_SHAPE, "n must be in [1, 16384]");
    if (k < 1 || k > n) return fail(CEM_E_SHAPE, "k must be in [1, n]");
    if (h < 1 || a < 1 || (long long)h * a > (1 << 20)) return fail(CEM_E_SHAPE, "bad h or a");
    if (ensure_select_ready() != CEM_OK) return CEM_E_HIP;
    return check_hip(cem::launch_select_refit(energy, actions, n, k, h * a, elite_idx, mu, sigma,
                                              static_cast<hipStream_t>(stream)),
                     "select/refit kernel");
  });
}

cem_status cem_sample(const float* mu, const float* sigma, int32_t n, int32_t h, int32_t a,
                      uint64_t seed, uint32_t round, uint32_t plan_id, float lo, float hi,
                      float* actions, uint32_t* raw_words, void* stream) {
  return guarded([&]() -> cem_status {
    if (!mu || !sigma || !actions) return fail(CEM_E_ARG, "null argument");
    if (!aligned(mu, 4) || !aligned(sigma, 4) || !aligned(actions, 4) || (raw_words && !aligned(raw_words, 4)))
      return fail(CEM_E_ARG, "misaligned pointer");
    if (n < 0 || h < 1 || a < 1 || (long long)n * h * a > (1LL << 31) - 4)
      return fail(CEM_E_SHAPE, "need n >= 0, h >= 1, a >= 1 and n*h*a < 2^31");
    if (!std::isfinite(lo) || !std::isfinite(hi) || lo > hi)
      return fail(CEM_E_ARG, "clamp bounds must be finite with lo <= hi");
    return check_hip(cem::launch_sample(mu, sigma, n, h * a, seed, round, plan_id, nullptr, lo, hi,
                                        actions, raw_words, static_cast<hipStream_t>(stream)),
                     "sampler kernel");
  });
}

cem_status cem_warm_start(const float* mu_prev, const float* sigma_prev, int32_t h, int32_t a,
                          float mu_fill, float sigma_fill, float sigma_floor, float* mu_next,
                          float* sigma_next, void* stream) {
  return guarded([&]() -> cem_status {
    if (!mu_prev || !sigma_prev || !mu_next || !sigma_next) return fail(CEM_E_ARG, "null argument");
    if (!aligned(mu_prev, 4) || !aligned(sigma_prev, 4) || !aligned(mu_next, 4) || !aligned(sigma_next, 4))
      return fail(CEM_E_ARG, "misaligned pointer");
    if (h < 1 || a < 1 || (long long)h * a > 1024) return fail(CEM_E_SHAPE, "need h >= 1, a >= 1, h * a <= 1024");
    if (!std::isfinite(mu_fill) || !std::isfinite(sigma_fill) || !(sigma_fill > 0.f) ||
        !std::isfinite(sigma_floor) || sigma_floor < 0.f)
      return fail(CEM_E_ARG, "need finite mu_fill, sigma_fill > 0 and finite sigma_floor >= 0");
    return check_hip(cem::launch_warm_start(mu_prev, sigma_prev, h, a, mu_fill, sigma_fill, sigma_floor,
                                            mu_next, sigma_next, static_cast<hipStream_t>(stream)),
                     "warm-start kernel");
  });
}

cem_status cem_fp8_quantize_rows(const float* x, int32_t rows, int32_t cols, uint8_t* codes,
                                 float* scale, void* stream) {
  return guarded([&]() -> cem_status {
    if (!x || !codes || !scale) return fail(CEM_E_ARG, "null argument");
    if (!aligned(x, 4) || !aligned(codes, 8) || !aligned(scale, 4)) return fail(CEM_E_ARG, "misaligned pointer");
    if (rows < 0 || cols < 8 || cols % 8 != 0 || (long long)rows * cols > (1LL << 31))
      return fail(CEM_E_SHAPE, "need rows >= 0, cols a positive multiple of 8, rows * cols <= 2^31");
    return check_hip(cem::launch_quantize_rows_fp8(x, rows, cols, codes, scale, static_cast<hipStream_t>(stream)),
                     "fp8 quantize kernel");
  });
}

cem_status topk_select(const float* energy, int32_t n, int32_t k, int32_t* idx, void* stream) {
  return guarded([&]() -> cem_status {
    if (!energy || !idx) return fail(CEM_E_ARG, "null argument");
    if (!aligned(energy, 4) || !aligned(idx, 4)) return fail(CEM_E_ARG, "misaligned pointer");
    if (n < 1 || n > cem::kMaxSelect) return fail(CEM_E_SHAPE, "n must be in [1, 16384]");
    if (k < 1 || k > n) return fail(CEM_E_SHAPE, "k must be in [1, n]");
    if (ensure_select_ready() != CEM_OK) return CEM_E_HIP;
    return check_hip(cem::launch_select_refit(energy, nullptr, n, k, 0, idx, nullptr, nullptr,
                                              static_cast<hipStream_t>(stream)),
                     "select kernel");
  });
}

cem_status cem_timer_enable(cem_model* model, int32_t enable) {
  return guarded([&]() -> cem_status {
    if (!model) return fail(CEM_E_ARG, "null model");
    if (enable != 0 && enable != 1) return fail(CEM_E_ARG, "enable must be 0 or 1");
    model->timers = enable == 1;
    model->ev_used = 0;
    return CEM_OK;
  });
}

cem_status cem_timer_read(cem_model* model, int64_t* launches, double* total_ms, double* total_flop) {
  return guarded([&]() -> cem_status {
    if (!model || !launches || !total_ms || !total_flop) return fail(CEM_E_ARG, "null argument");
    return finish(cem::timer_read(model, launches, total_ms, total_flop));
  });
}

}  // extern "C"
