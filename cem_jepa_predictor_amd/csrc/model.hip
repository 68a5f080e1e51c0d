// Host orchestration of the predictor rollout and the CEM plan step.
//
// Page "Real-Time Inference for JEPA World Model Architectures with Ray":
//  * section 01: a planning step encodes frame and goal once, then runs ten
//    sequential rounds of sample -> predict -> score -> keep best -> refit;
//  * section 04: the latents stay resident for the whole plan; each round only
//    moves candidate actions and energies;
//  * section 05: the predictor is frame-causal (KV cache across steps).
// Here every round runs on one GPU stream with no host synchronisation: the
// frame projection of z_obs is computed once per plan, the round's samples,
// energies and refit live in device buffers, and the whole R-round sequence
// is captured once per shape as a HIP graph and replayed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "model.hpp"

// Plan state of cem_plan_noalloc: one copy of this array on every device the
// library runs on, for callers that cannot allocate.  In host code `scratch`
// names a host-side stand-in, not a device address; the address of a device's
// copy comes from hipGetSymbolAddress, taken once per device when a model is
// created there (scratch_setup below), and only that address is used.
static __device__ __align__(256) uint8_t scratch[cem::kPlanScratchBytes];

namespace cem {

Status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return Status::Ok();
  Status s;
  s.code = (e == hipErrorOutOfMemory) ? CEM_E_OOM : CEM_E_HIP;
  s.msg = std::string(what) + ": " + hipGetErrorString(e);
  return s;
}

#define CEM_TRY(expr, what)                               \
  do {                                                    \
    hipError_t _e = (expr);                               \
    if (_e != hipSuccess) return hip_status(_e, (what));  \
  } while (0)

DeviceGuard::DeviceGuard(int device) {
  if (hipGetDevice(&prev) != hipSuccess) prev = -1;
  if (prev != device) (void)hipSetDevice(device);
}
DeviceGuard::~DeviceGuard() {
  int cur = -1;
  if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
}

namespace {

uint16_t host_bf16(float f) {   // round to nearest even (finite inputs)
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// OCP e4m3 code of a finite float with |v| <= 448, rounded to nearest, ties to the
// even mantissa: 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormals below 2^-6.
uint8_t host_e4m3(float v) {
  const uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  const double a = std::fabs((double)v);
  if (a == 0.0) return sign;
  int ex = 0;
  std::frexp(a, &ex);                         // a in [2^(ex-1), 2^ex)
  int e = std::max(ex - 1, -6);
  double m = std::nearbyint(std::ldexp(a, -(e - 3)));   // round half to even (default mode)
  if (m >= 16.0) { m = 8.0; ++e; }
  if (m < 8.0) return (uint8_t)(sign | (uint8_t)m);     // subnormal (e == -6)
  return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((int)m - 8)));
}

// Bump layout over one allocation.
struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  }
};

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices] = {};

// Record the current device's copy of `scratch` (the device must be current).
hipError_t scratch_setup(int device) {
  if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device]) return hipSuccess;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch[device] = ptr;
  return hipSuccess;
}

void* scratch_of(int device) {
  if (device < 0 || device >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[device];
}

// Offsets of the plan state for n candidates, k elites, r rounds, ha = H * A,
// nb problems, carved from one block of device memory.
struct PlanLayout {
  size_t x, e, mu, sg, el, zo, zg, s0, zt, f0, pp, bytes;
};

PlanLayout plan_layout(const cem_model* m, int n, int k, int r, int ha, int nb) {
  const size_t P = m->desc.patches, PE = P * m->desc.enc_dim, PD = P * m->desc.d_model;
  Layout l;
  PlanLayout o;
  o.x = l.take((size_t)r * nb * n * ha * 4);
  o.e = l.take((size_t)r * nb * n * 4);
  o.mu = l.take((size_t)(r + 1) * nb * ha * 4);
  o.sg = l.take((size_t)(r + 1) * nb * ha * 4);
  o.el = l.take((size_t)r * nb * k * 4);
  o.zo = l.take(nb * PE * 4);
  o.zg = l.take(nb * PE * 4);
  o.s0 = l.take((size_t)nb * 64 * 4);
  o.zt = l.take(nb * PE * m->esz);
  o.f0 = l.take(nb * PD * m->esz);
  o.pp = l.take(16);
  o.bytes = l.off;
  return o;
}

void carve_plan_state(PlanState& ps, void* base, const PlanLayout& o) {
  uint8_t* b = static_cast<uint8_t*>(base);
  ps.x_hist = (float*)(b + o.x); ps.e_hist = (float*)(b + o.e);
  ps.mu_hist = (float*)(b + o.mu); ps.sigma_hist = (float*)(b + o.sg);
  ps.elites = (int*)(b + o.el);
  ps.zobs = (float*)(b + o.zo); ps.zgoal = (float*)(b + o.zg); ps.s0 = (float*)(b + o.s0);
  ps.zobs_t = b + o.zt; ps.f0 = b + o.f0;
  ps.params = (uint32_t*)(b + o.pp);
}

}  // namespace

size_t weights_count(const cem_model_desc& d) {
  const size_t D = d.d_model, F = d.d_mlp, E = d.enc_dim, A = d.action_dim, S = d.state_dim;
  const size_t per_layer = 2 * D + D * 3 * D + 3 * D + D * D + D + 2 * D + D * F + F + F * D + D;
  return E * D + D + A * D + D + S * D + D + (size_t)d.layers * per_layer + 2 * D + D * E + E;
}

Status validate_desc(const cem_model_desc& d) {
  auto bad = [](cem_status c, const std::string& m) { Status s; s.code = c; s.msg = m; return s; };
  if (d.dtype != CEM_F32 && d.dtype != CEM_BF16 && d.dtype != CEM_FP8)
    return bad(CEM_E_DTYPE, "dtype must be CEM_F32, CEM_BF16 or CEM_FP8");
  if (d.dtype == CEM_FP8 && d.d_model % 512 != 0)
    return bad(CEM_E_SHAPE, "fp8 models need d_model % 512 == 0");
  if (d.layers < 1 || d.layers > 256) return bad(CEM_E_SHAPE, "layers must be in [1, 256]");
  if (d.heads < 1 || d.d_model < 1 || d.d_model % d.heads != 0)
    return bad(CEM_E_SHAPE, "d_model must be a positive multiple of heads");
  if (!layernorm_supports(d.d_model))
    return bad(CEM_E_SHAPE, "d_model must be one of 128, 256, 384, 512, 768, 1024, 1536, 2048, 4096");
  if (d.d_mlp < 64 || d.d_mlp % 64 != 0 || d.d_mlp > 65536) return bad(CEM_E_SHAPE, "d_mlp must be a multiple of 64");
  if (d.enc_dim < 64 || d.enc_dim % 64 != 0 || d.enc_dim > 65536) return bad(CEM_E_SHAPE, "enc_dim must be a multiple of 64");
  if (d.patches < 1 || d.patches > 4096) return bad(CEM_E_SHAPE, "patches must be in [1, 4096]");
  if (d.action_dim < 1 || d.action_dim > 32 || d.state_dim < 1 || d.state_dim > 32)
    return bad(CEM_E_SHAPE, "action_dim and state_dim must be in [1, 32]");
  if (d.max_horizon < 1 || d.max_horizon > kMaxBlocks) return bad(CEM_E_SHAPE, "max_horizon must be in [1, 8]");
  if (d.max_horizon > 1 && d.state_dim != d.action_dim)
    return bad(CEM_E_SHAPE, "horizon > 1 advances the state by the action: state_dim must equal action_dim");
  if (d.max_samples < 1 || d.max_samples > kMaxSelect) return bad(CEM_E_SHAPE, "max_samples must be in [1, 16384]");
  if (!(d.ln_eps > 0.f) || !std::isfinite(d.ln_eps)) return bad(CEM_E_ARG, "ln_eps must be positive and finite");
  const int dh = d.d_model / d.heads, B = d.patches + 2;
  if (d.dtype != CEM_F32 && !attention_bf16_supports(dh, B))
    return bad(CEM_E_SHAPE, "bf16 attention needs head dim 64 and patches + 2 <= 320");
  if (d.dtype == CEM_F32 && !attention_f32_supports(dh))
    return bad(CEM_E_SHAPE, "fp32 attention needs head dim 16, 32, 64 or 128");
  const long long rows = (long long)d.max_samples * B;
  if (rows * std::max({3LL * d.d_model, (long long)d.d_mlp, (long long)d.enc_dim}) > (1LL << 40))
    return bad(CEM_E_SHAPE, "workspace too large");
  if (rows > (1LL << 30)) return bad(CEM_E_SHAPE, "max_samples * (patches + 2) too large");
  return Status::Ok();
}

Status model_create(const cem_model_desc& d, const float* host_w, int device, cem_model** out) {
  Status v = validate_desc(d);
  if (!v.ok()) return v;
  int ndev = 0;
  CEM_TRY(hipGetDeviceCount(&ndev), "hipGetDeviceCount");
  if (device < 0 || device >= ndev) {
    Status s; s.code = CEM_E_ARG; s.msg = "device index out of range"; return s;
  }
  DeviceGuard guard(device);
  cem_model* m = new cem_model();
  m->desc = d;
  m->device = device;
  m->bf16 = d.dtype != CEM_F32;
  m->fp8 = d.dtype == CEM_FP8;
  m->ln_fold = d.dtype == CEM_BF16;
  m->esz = m->bf16 ? 2 : 4;
  m->B = d.patches + 2;
  m->rows_max = (long long)d.max_samples * m->B;

  const size_t D = d.d_model, F = d.d_mlp, E = d.enc_dim, A = d.action_dim, S = d.state_dim;
  const size_t L = d.layers, P = d.patches, es = m->esz;

  // ---- weights: host staging in device layout, then one upload
  Layout wl;
  const size_t o_w_in = wl.take(D * E * es), o_b_in = wl.take(D * 4);
  const size_t o_w_a = wl.take(A * D * 4), o_b_a = wl.take(D * 4);
  const size_t o_w_s = wl.take(S * D * 4), o_b_s = wl.take(D * 4);
  struct LO {
    size_t ln1_g, ln1_b, w_qkv, b_qkv, w_o, b_o, ln2_g, ln2_b, w_1, b_1, w_2, b_2;
  };
  std::vector<LO> lo(L);
  const size_t fold = m->ln_fold ? 1 : 0;
  for (size_t l = 0; l < L; ++l) {
    lo[l].ln1_g = wl.take(D * 4); lo[l].ln1_b = wl.take(D * 4);
    const size_t es8 = m->fp8 ? 1 : es;   // fp8 models: e4m3 codes for q|k|v and MLP up
    lo[l].w_qkv = wl.take(3 * D * D * es8); lo[l].b_qkv = wl.take((1 + fold) * 3 * D * 4);
    lo[l].w_o = wl.take(D * D * es); lo[l].b_o = wl.take(D * 4);
    lo[l].ln2_g = wl.take(D * 4); lo[l].ln2_b = wl.take(D * 4);
    lo[l].w_1 = wl.take(F * D * es8); lo[l].b_1 = wl.take((1 + fold) * F * 4);
    lo[l].w_2 = wl.take(D * F * es); lo[l].b_2 = wl.take(D * 4);
  }
  const size_t o_lnf_g = wl.take(D * 4), o_lnf_b = wl.take(D * 4);
  const size_t o_w_out = wl.take(E * D * es), o_b_out = wl.take(E * 4);

  std::vector<uint8_t> hw;
  try {
    hw.assign(wl.off, 0);
  } catch (const std::bad_alloc&) {
    delete m;
    Status s; s.code = CEM_E_OOM; s.msg = "host staging buffer"; return s;
  }
  const float* src = host_w;
  auto put_vec = [&](size_t off, size_t count) {
    std::memcpy(hw.data() + off, src, count * 4);
    src += count;
  };
  // matrix stored [in, out] in the flat buffer -> [out, in] (K contiguous) in model dtype
  auto put_mat_t = [&](size_t off, size_t in, size_t outd) {
    for (size_t i = 0; i < in; ++i)
      for (size_t o = 0; o < outd; ++o) {
        const float v = src[i * outd + o];
        const size_t dst = o * in + i;
        if (m->bf16) {
          const uint16_t b = host_bf16(v);
          std::memcpy(hw.data() + off + dst * 2, &b, 2);
        } else {
          std::memcpy(hw.data() + off + dst * 4, &v, 4);
        }
      }
    src += in * outd;
  };
  // fp8: one scale for the whole matrix, ws = amax / 448; codes = e4m3(clamp(v * (448 /
  // amax), +-448)); the bias that follows is stored divided by ws
  std::vector<float> ws_qkv(L, 1.f), ws_1(L, 1.f);
  auto put_mat_t8 = [&](size_t off, size_t in, size_t outd, float& ws) {
    float amax = 0.f;
    for (size_t i = 0; i < in * outd; ++i) amax = std::max(amax, std::fabs(src[i]));
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    ws = amax > 0.f ? amax / 448.0f : 1.0f;
    for (size_t i = 0; i < in; ++i)
      for (size_t o = 0; o < outd; ++o) {
        const float y = std::min(std::max(src[i * outd + o] * inv, -448.0f), 448.0f);
        hw[off + o * in + i] = host_e4m3(y);
      }
    src += in * outd;
  };
  // LayerNorm fold (x - mean) rstd gamma W + beta W + b = rstd (x W' - mean 1^T W') + b'
  // with W' = diag(gamma) W: stores bf16(W') transposed, and at b_off b' = b + beta W
  // (from the unrounded W) followed by the column sums of the bf16 W' values (so the
  // mean term cancels exactly what the GEMM contracts).  gamma and beta are the `in`
  // values just before the matrix in the flat buffer.
  auto put_mat_t_folded = [&](size_t off, size_t in, size_t outd, size_t b_off) {
    const size_t cs_off = b_off + outd * 4;
    const float* g = src - 2 * in;
    const float* beta = src - in;
    const float* bias = src + in * outd;
    std::vector<double> cs(outd, 0.0), bb(outd, 0.0);
    for (size_t i = 0; i < in; ++i)
      for (size_t o = 0; o < outd; ++o) {
        const float v = src[i * outd + o];
        const uint16_t b = host_bf16(g[i] * v);
        std::memcpy(hw.data() + off + (o * in + i) * 2, &b, 2);
        uint32_t u = (uint32_t)b << 16;
        float f;
        std::memcpy(&f, &u, 4);
        cs[o] += (double)f;
        bb[o] += (double)beta[i] * (double)v;
      }
    for (size_t o = 0; o < outd; ++o) {
      const float c = (float)cs[o], bo = (float)((double)bias[o] + bb[o]);
      std::memcpy(hw.data() + cs_off + o * 4, &c, 4);
      std::memcpy(hw.data() + b_off + o * 4, &bo, 4);
    }
    src += in * outd + outd;   // the matrix and its bias
  };
  auto put_vec_scaled = [&](size_t off, size_t count, float ws) {
    for (size_t i = 0; i < count; ++i) {
      const float v = src[i] / ws;
      std::memcpy(hw.data() + off + i * 4, &v, 4);
    }
    src += count;
  };
  put_mat_t(o_w_in, E, D); put_vec(o_b_in, D);
  put_vec(o_w_a, A * D); put_vec(o_b_a, D);
  put_vec(o_w_s, S * D); put_vec(o_b_s, D);
  for (size_t l = 0; l < L; ++l) {
    put_vec(lo[l].ln1_g, D); put_vec(lo[l].ln1_b, D);
    if (m->fp8) { put_mat_t8(lo[l].w_qkv, D, 3 * D, ws_qkv[l]); put_vec_scaled(lo[l].b_qkv, 3 * D, ws_qkv[l]); }
    else if (m->ln_fold) put_mat_t_folded(lo[l].w_qkv, D, 3 * D, lo[l].b_qkv);
    else { put_mat_t(lo[l].w_qkv, D, 3 * D); put_vec(lo[l].b_qkv, 3 * D); }
    put_mat_t(lo[l].w_o, D, D); put_vec(lo[l].b_o, D);
    put_vec(lo[l].ln2_g, D); put_vec(lo[l].ln2_b, D);
    if (m->fp8) { put_mat_t8(lo[l].w_1, D, F, ws_1[l]); put_vec_scaled(lo[l].b_1, F, ws_1[l]); }
    else if (m->ln_fold) put_mat_t_folded(lo[l].w_1, D, F, lo[l].b_1);
    else { put_mat_t(lo[l].w_1, D, F); put_vec(lo[l].b_1, F); }
    put_mat_t(lo[l].w_2, F, D); put_vec(lo[l].b_2, D);
  }
  put_vec(o_lnf_g, D); put_vec(o_lnf_b, D);
  put_mat_t(o_w_out, D, E); put_vec(o_b_out, E);

  auto fail = [&](Status s) { model_destroy(m); return s; };
  hipError_t e = hipMalloc(&m->warena, wl.off);
  if (e != hipSuccess) return fail(hip_status(e, "hipMalloc(weights)"));
  e = hipMemcpy(m->warena, hw.data(), wl.off, hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(hip_status(e, "hipMemcpy(weights)"));
  uint8_t* wb = static_cast<uint8_t*>(m->warena);
  m->w_in_t = wb + o_w_in; m->b_in = (float*)(wb + o_b_in);
  m->w_a = (float*)(wb + o_w_a); m->b_a = (float*)(wb + o_b_a);
  m->w_s = (float*)(wb + o_w_s); m->b_s = (float*)(wb + o_b_s);
  m->layers.resize(L);
  for (size_t l = 0; l < L; ++l) {
    LayerW& w = m->layers[l];
    w.ln1_g = (float*)(wb + lo[l].ln1_g); w.ln1_b = (float*)(wb + lo[l].ln1_b);
    w.w_qkv_t = wb + lo[l].w_qkv; w.b_qkv = (float*)(wb + lo[l].b_qkv);
    w.w_o_t = wb + lo[l].w_o; w.b_o = (float*)(wb + lo[l].b_o);
    w.ln2_g = (float*)(wb + lo[l].ln2_g); w.ln2_b = (float*)(wb + lo[l].ln2_b);
    w.w_1_t = wb + lo[l].w_1; w.b_1 = (float*)(wb + lo[l].b_1);
    w.w_2_t = wb + lo[l].w_2; w.b_2 = (float*)(wb + lo[l].b_2);
    w.ws_qkv = ws_qkv[l]; w.ws_1 = ws_1[l];
  }
  m->lnf_g = (float*)(wb + o_lnf_g); m->lnf_b = (float*)(wb + o_lnf_b);
  m->w_out_t = wb + o_w_out; m->b_out = (float*)(wb + o_b_out);

  // ---- workspace
  const size_t rows = (size_t)m->rows_max;
  const size_t kv_slots = L * (size_t)(d.max_horizon - 1) + 1;
  Layout al;
  const size_t o_x = al.take(rows * D * es), o_h = al.take(rows * D * es), o_q = al.take(rows * D * es);
  const size_t o_u = al.take(rows * F * es);
  const size_t o_kv = al.take(kv_slots * rows * 2 * D * es);
  const size_t o_zhat = al.take((size_t)d.max_samples * P * E * es);
  const size_t o_f0 = al.take(P * D * es), o_zobs = al.take(P * E * es);
  const size_t o_h8 = al.take(m->fp8 ? rows * D : 0), o_hs = al.take(m->fp8 ? rows * 4 : 0);
  const size_t o_stats = al.take(fold * 2 * rows * 4);
  // residual GEMMs write LN statistics (their launcher takes up to 2^28 rows)
  const size_t parts = (fold && D % 256 == 0 && rows < (size_t(1) << 28)) ? 1 : 0;
  const size_t o_parts = al.take(parts * (D / 64) * rows * 8);
  e = hipMalloc(&m->arena, al.off);
  if (e != hipSuccess) return fail(hip_status(e, "hipMalloc(workspace)"));
  uint8_t* ab = static_cast<uint8_t*>(m->arena);
  m->x = ab + o_x; m->h = ab + o_h; m->q = ab + o_q; m->u = ab + o_u; m->kv = ab + o_kv;
  m->zhat = ab + o_zhat; m->f0 = ab + o_f0; m->zobs_t = ab + o_zobs;
  if (m->fp8) { m->h8 = ab + o_h8; m->hs = reinterpret_cast<float*>(ab + o_hs); }
  if (m->ln_fold) m->ln_stats = reinterpret_cast<float*>(ab + o_stats);
  if (parts) m->ln_parts = reinterpret_cast<float*>(ab + o_parts);

  e = select_init();
  if (e != hipSuccess) return fail(hip_status(e, "select_init"));
  e = gemm_init();
  if (e != hipSuccess) return fail(hip_status(e, "gemm_init"));
  e = attention_init();
  if (e != hipSuccess) return fail(hip_status(e, "attention_init"));
  e = scratch_setup(device);
  if (e != hipSuccess) return fail(hip_status(e, "hipGetSymbolAddress(scratch)"));
  e = hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking);
  if (e != hipSuccess) return fail(hip_status(e, "hipStreamCreate"));
  *out = m;
  return Status::Ok();
}

void model_destroy(cem_model* m) {
  if (!m) return;
  DeviceGuard guard(m->device);
  (void)hipDeviceSynchronize();
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  for (auto& pr : m->ev) { (void)hipEventDestroy(pr.first); (void)hipEventDestroy(pr.second); }
  if (m->plan.mem) (void)hipFree(m->plan.mem);
  if (m->arena) (void)hipFree(m->arena);
  if (m->warena) (void)hipFree(m->warena);
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  delete m;
}

namespace {

// ---------------------------------------------------------------- timers
hipError_t timer_start(cem_model* m, hipStream_t st, double flop) {
  if (!m->timers) return hipSuccess;
  if (m->ev_used == m->ev.size()) {
    std::pair<hipEvent_t, hipEvent_t> pr;
    hipError_t e = hipEventCreate(&pr.first);
    if (e != hipSuccess) return e;
    e = hipEventCreate(&pr.second);
    if (e != hipSuccess) return e;
    m->ev.push_back(pr);
    m->ev_flop.push_back(0.0);
  }
  m->ev_flop[m->ev_used] = flop;
  return hipEventRecord(m->ev[m->ev_used].first, st);
}
hipError_t timer_stop(cem_model* m, hipStream_t st) {
  if (!m->timers) return hipSuccess;
  return hipEventRecord(m->ev[m->ev_used++].second, st);
}

hipError_t gemm(cem_model* m, const void* A, int lda, const void* Bt, int ldb, int M, int N, int K,
                const Epilogue& e, hipStream_t st) {
  hipError_t r = timer_start(m, st, 2.0 * M * (double)N * K);
  if (r != hipSuccess) return r;
  r = m->bf16 ? launch_gemm_bf16(static_cast<const bf16*>(A), lda, static_cast<const bf16*>(Bt),
                                 ldb, M, N, K, e, st)
              : launch_gemm_f32(static_cast<const float*>(A), lda,
                                static_cast<const float*>(Bt), ldb, M, N, K, e, st);
  if (r != hipSuccess) return r;
  return timer_stop(m, st);
}

hipError_t gemm8(cem_model* m, const uint8_t* A, int lda, const void* Bt, int ldb, int M, int N,
                 int K, const float* row_scale, float w_scale, const Epilogue& e, hipStream_t st) {
  hipError_t r = timer_start(m, st, 2.0 * M * (double)N * K);
  if (r != hipSuccess) return r;
  r = launch_gemm_fp8(A, lda, static_cast<const uint8_t*>(Bt), ldb, M, N, K, row_scale, w_scale, e, st);
  if (r != hipSuccess) return r;
  return timer_stop(m, st);
}

// bf16 GEMM over M raw residual rows with the LayerNorm before it folded in: row
// statistics of those rows (combined from the partial statistics of the residual
// GEMM that wrote them when `from_parts`, else read from the rows), then the GEMM
// with rstd / mean row terms and the folded bias / column-sum terms (e.bias, 2 N floats)
hipError_t gemm_ln(cem_model* m, const void* A, int lda, const void* Bt, int ldb, int M, int N, int K,
                   const Epilogue& e, bool from_parts, hipStream_t st) {
  hipError_t r = from_parts ? launch_row_stats_combine(m->ln_parts, M, K, m->desc.ln_eps, m->ln_stats + M,
                                                       m->ln_stats, st)
                            : launch_row_stats(static_cast<const bf16*>(A), M, K, m->desc.ln_eps,
                                               m->ln_stats + M, m->ln_stats, st);
  if (r != hipSuccess) return r;
  r = timer_start(m, st, 2.0 * M * (double)N * K);
  if (r != hipSuccess) return r;
  r = launch_gemm_bf16_rows(static_cast<const bf16*>(A), lda, static_cast<const bf16*>(Bt), ldb, M,
                            N, K, m->ln_stats, e, st);
  if (r != hipSuccess) return r;
  return timer_stop(m, st);
}

Epilogue epi(const float* bias, void* c0, int ld0, int split, void* c1 = nullptr, int ld1 = 0,
             int gelu = 0, int residual = 0, RowMap rows = RowMap::identity(), float* stats = nullptr) {
  Epilogue e;
  e.bias = bias; e.c0 = c0; e.c1 = c1; e.ld0 = ld0; e.ld1 = ld1; e.split = split;
  e.gelu = gelu; e.residual = residual; e.rows = rows; e.stats = stats;
  return e;
}

void* kv_slot(cem_model* m, int l, int tau, int horizon) {
  const size_t slot = (tau < horizon - 1) ? (size_t)l * (m->desc.max_horizon - 1) + tau
                                          : (size_t)m->desc.layers * (m->desc.max_horizon - 1);
  return static_cast<uint8_t*>(m->kv) + slot * (size_t)m->rows_max * 2 * m->desc.d_model * m->esz;
}

// Layer 0 of the first frame block at horizon 1 (bf16 models with the LayerNorm folded,
// and fp8-projection models): every candidate of a problem shares that problem's state
// token and frame tokens (rows 1 .. B-1), so their LayerNorm statistics and q|k|v
// projection are the same rows computed n_per times over.  They are computed once per
// problem instead, and each candidate's action row once, in one compact block of
// problems (B - 1) + n rows that the attention reads q, k and v from.  Every row goes
// through the same kernels and arithmetic as in the full batch, so the results are
// unchanged bit for bit.  Horizon > 1 keeps the full layer-0 K/V of the first block in
// the KV cache for later steps.
bool layer0_compact(const cem_model* m, int n, int n_per, int H) {
  if (!(m->ln_fold || m->fp8) || H != 1 || n_per <= 0 || n % n_per != 0 || m->B < 2) return false;
  const long long rows = (long long)(n / n_per) * (m->B - 1) + n;
  // compact rows go to the q buffer ([rows_max, d]) and their q|k|v to the current KV slot
  // ([rows_max, 2 d]); the attention addresses that block with 32-bit byte offsets
  return rows <= m->rows_max && rows * 3 <= (long long)m->rows_max * 2 &&
         rows * 3 * m->desc.d_model * 2 < 0x7ffffff0LL;
}

// f0 = z_obs W_in + b_in for each of `problems` observations [problems, P, E],
// shared by every candidate's first frame block of that problem.
template <typename T>
hipError_t enqueue_frame0(cem_model* m, const float* z_obs, int problems, void* zobs_t, void* f0,
                          hipStream_t st) {
  const int P = m->desc.patches, E = m->desc.enc_dim, D = m->desc.d_model;
  // stage z_obs (caller memory, 4-byte aligned) into the aligned model-dtype buffer
  hipError_t r = launch_convert<T>(z_obs, static_cast<T*>(zobs_t), (long long)problems * P * E, st);
  if (r != hipSuccess) return r;
  return gemm(m, zobs_t, E, m->w_in_t, E, problems * P, D, E, epi(m->b_in, f0, D, D), st);
}

// Autoregressive block-causal rollout of n candidates; leaves z_H in m->zhat.
// Candidate i belongs to problem i / n_per: state s0 + (i / n_per) S, frame-0
// tokens f0 + (i / n_per) P d.
template <typename T>
hipError_t enqueue_rollout(cem_model* m, const float* X, int n, int H, const float* s0,
                           const void* f0, int n_per, hipStream_t st) {
  const cem_model_desc& d = m->desc;
  const int B = m->B, P = d.patches, D = d.d_model, F = d.d_mlp, E = d.enc_dim;
  const int rows = n * B;
  hipError_t r;
#define RUN(x) do { r = (x); if (r != hipSuccess) return r; } while (0)
  for (int t = 0; t < H; ++t) {
    RUN(launch_embed_action_state<T>(X, n, H, t, d.action_dim, d.state_dim, s0, m->w_a, m->b_a,
                                     m->w_s, m->b_s, static_cast<T*>(m->x), B, D, n_per, st));
    if (t == 0) {
      RUN(launch_broadcast_frame<T>(static_cast<const T*>(f0), P, D, static_cast<T*>(m->x), n, B,
                                    n_per, st));
    } else {
      // frame rows of block t = previous prediction projected in (row r -> n B + 2 + p)
      RUN(gemm(m, m->zhat, E, m->w_in_t, E, n * P, D, E,
               epi(m->b_in, m->x, D, D, nullptr, 0, 0, 0, RowMap{P, B, 2}), st));
    }
    for (int l = 0; l < d.layers; ++l) {
      const LayerW& w = m->layers[l];
      void* qkv_c = nullptr;   // compact layer-0 q|k|v block (layer0_compact)
      if (l == 0 && t == 0 && layer0_compact(m, n, n_per, H)) {
        const int problems = n / n_per, rc = problems * (B - 1) + n;
        bf16* const xc = static_cast<bf16*>(m->q);
        qkv_c = kv_slot(m, 0, 0, H);
        RUN(launch_gather_layer0(static_cast<const bf16*>(m->x), B, D, problems, n_per, n, xc, st));
        if (m->fp8) {
          RUN(launch_layernorm_fp8(xc, rc, D, RowMap::identity(), w.ln1_g, w.ln1_b, d.ln_eps, m->h8,
                                   m->hs, st));
          RUN(gemm8(m, m->h8, D, w.w_qkv_t, D, rc, 3 * D, D, m->hs, w.ws_qkv,
                    epi(w.b_qkv, qkv_c, 3 * D, 3 * D), st));
        } else {
          RUN(launch_row_stats(xc, rc, D, d.ln_eps, m->ln_stats + rc, m->ln_stats, st));
          RUN(timer_start(m, st, 2.0 * rc * (3.0 * D) * D));
          RUN(launch_gemm_bf16_rows(xc, D, static_cast<const bf16*>(w.w_qkv_t), D, rc, 3 * D, D,
                                    m->ln_stats, epi(w.b_qkv, qkv_c, 3 * D, 3 * D), st));
          RUN(timer_stop(m, st));
        }
      } else if (m->fp8) {
        RUN(launch_layernorm_fp8(static_cast<const bf16*>(m->x), rows, D, RowMap::identity(), w.ln1_g,
                                 w.ln1_b, d.ln_eps, m->h8, m->hs, st));
        RUN(gemm8(m, m->h8, D, w.w_qkv_t, D, rows, 3 * D, D, m->hs, w.ws_qkv,
                  epi(w.b_qkv, m->q, D, D, kv_slot(m, l, t, H), 2 * D), st));
      } else if (m->ln_fold) {
        // layer 0's input rows come from the token embedding, the others' from a residual GEMM
        RUN(gemm_ln(m, m->x, D, w.w_qkv_t, D, rows, 3 * D, D,
                    epi(w.b_qkv, m->q, D, D, kv_slot(m, l, t, H), 2 * D), l > 0 && m->ln_parts, st));
      } else {
        RUN(launch_layernorm<T>(static_cast<const T*>(m->x), rows, D, RowMap::identity(), w.ln1_g,
                                w.ln1_b, d.ln_eps, static_cast<T*>(m->h), st));
        RUN(gemm(m, m->h, D, w.w_qkv_t, D, rows, 3 * D, D,
                 epi(w.b_qkv, m->q, D, D, kv_slot(m, l, t, H), 2 * D), st));
      }
      AttnArgs a{};
      a.q = m->q; a.ldq = D;
      for (int tau = 0; tau <= t; ++tau) a.kv[tau] = kv_slot(m, l, tau, H);
      a.ldkv = 2 * D; a.o = m->h; a.ldo = D;
      a.n = n; a.heads = d.heads; a.dh = D / d.heads; a.d = D; a.B = B; a.nblk = t + 1;
      a.scale = 1.0f / std::sqrt((float)a.dh);
      if (qkv_c) {
        a.qkv_c = qkv_c; a.c_problems = n / n_per; a.c_n_per = n_per;
        qkv_c = nullptr;
      }
      RUN(m->bf16 ? launch_attention_bf16(a, st) : launch_attention_f32(a, st));
      RUN(gemm(m, m->h, D, w.w_o_t, D, rows, D, D,
               epi(w.b_o, m->x, D, D, nullptr, 0, 0, 1, RowMap::identity(), m->ln_parts), st));
      if (m->fp8) {
        RUN(launch_layernorm_fp8(static_cast<const bf16*>(m->x), rows, D, RowMap::identity(), w.ln2_g,
                                 w.ln2_b, d.ln_eps, m->h8, m->hs, st));
        RUN(gemm8(m, m->h8, D, w.w_1_t, D, rows, F, D, m->hs, w.ws_1,
                  epi(w.b_1, m->u, F, F, nullptr, 0, 1, 0), st));
      } else if (m->ln_fold) {
        RUN(gemm_ln(m, m->x, D, w.w_1_t, D, rows, F, D, epi(w.b_1, m->u, F, F, nullptr, 0, 1, 0),
                    m->ln_parts != nullptr, st));
      } else {
        RUN(launch_layernorm<T>(static_cast<const T*>(m->x), rows, D, RowMap::identity(), w.ln2_g,
                                w.ln2_b, d.ln_eps, static_cast<T*>(m->h), st));
        RUN(gemm(m, m->h, D, w.w_1_t, D, rows, F, D, epi(w.b_1, m->u, F, F, nullptr, 0, 1, 0), st));
      }
      // the last layer's rows go to the final LayerNorm, which computes its own statistics
      RUN(gemm(m, m->u, F, w.w_2_t, F, rows, D, F,
               epi(w.b_2, m->x, D, D, nullptr, 0, 0, 1, RowMap::identity(),
                   l + 1 < d.layers ? m->ln_parts : nullptr), st));
    }
    // final LayerNorm of the patch rows, then the out-projection to the encoder width
    RUN(launch_layernorm<T>(static_cast<const T*>(m->x), n * P, D, RowMap{P, B, 2}, m->lnf_g,
                            m->lnf_b, d.ln_eps, static_cast<T*>(m->h), st));
    RUN(gemm(m, m->h, D, m->w_out_t, D, n * P, E, D, epi(m->b_out, m->zhat, E, E), st));
  }
#undef RUN
  return hipSuccess;
}

template <typename T>
hipError_t enqueue_plan_body(cem_model* m, const PlanState& ps, const cem_params& p, int batch,
                             hipStream_t st) {
  const int N = p.n_samples, K = p.n_elites, H = p.horizon, ha = H * m->desc.action_dim;
  const int NB = batch * N;
  const long long pe = (long long)m->desc.patches * m->desc.enc_dim;
  hipError_t r = enqueue_frame0<T>(m, ps.zobs, batch, ps.zobs_t, ps.f0, st);
  if (r != hipSuccess) return r;
  for (int rd = 0; rd < p.rounds; ++rd) {
    float* x = ps.x_hist + (size_t)rd * NB * ha;
    float* mu_rd = ps.mu_hist + (size_t)rd * batch * ha;
    float* sg_rd = ps.sigma_hist + (size_t)rd * batch * ha;
    r = launch_sample(mu_rd, sg_rd, N, ha, p.seed, (uint32_t)rd, p.plan_id, ps.params, p.clamp_lo,
                      p.clamp_hi, x, nullptr, st, batch);
    if (r != hipSuccess) return r;
    r = enqueue_rollout<T>(m, x, NB, H, ps.s0, ps.f0, N, st);
    if (r != hipSuccess) return r;
    r = launch_energy<T>(static_cast<const T*>(m->zhat), ps.zgoal, NB, pe, ps.e_hist + (size_t)rd * NB, N, st);
    if (r != hipSuccess) return r;
    r = launch_select_refit(ps.e_hist + (size_t)rd * NB, x, N, K, ha, ps.elites + (size_t)rd * batch * K,
                            mu_rd + (size_t)batch * ha, sg_rd + (size_t)batch * ha, st, batch);
    if (r != hipSuccess) return r;
  }
  return hipSuccess;
}

Status ensure_plan_state(cem_model* m, const cem_params& p, int batch) {
  PlanState& ps = m->plan;
  const int ha = p.horizon * m->desc.action_dim;
  if (ps.mem && p.n_samples <= ps.n && p.n_elites <= ps.k && p.rounds <= ps.r && ha <= ps.ha &&
      batch <= ps.batch)
    return Status::Ok();
  const int n = std::max(p.n_samples, ps.n), k = std::max(p.n_elites, ps.k);
  const int r = std::max(p.rounds, ps.r), hh = std::max(ha, ps.ha), nb = std::max(batch, ps.batch);
  const PlanLayout l = plan_layout(m, n, k, r, hh, nb);
  // existing graphs reference the old buffers
  CEM_TRY(hipDeviceSynchronize(), "hipDeviceSynchronize");
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  m->graphs.clear();
  if (ps.mem) { (void)hipFree(ps.mem); ps.mem = nullptr; }
  CEM_TRY(hipMalloc(&ps.mem, l.bytes), "hipMalloc(plan state)");
  ps.n = n; ps.k = k; ps.r = r; ps.ha = hh; ps.batch = nb;
  carve_plan_state(ps, ps.mem, l);
  return Status::Ok();
}

template <typename T>
Status run_plan(cem_model* m, const cem_params& p, int batch, hipStream_t st) {
  const PlanState& ps = m->plan;
  if (!p.use_graph || m->timers) return hip_status(enqueue_plan_body<T>(m, ps, p, batch, st), "plan kernels");
  uint32_t lo_bits, hi_bits;
  std::memcpy(&lo_bits, &p.clamp_lo, 4);
  std::memcpy(&hi_bits, &p.clamp_hi, 4);
  const GraphKey key{p.n_samples, p.n_elites, p.rounds, p.horizon, lo_bits, hi_bits, batch};
  auto it = m->graphs.find(key);
  if (it == m->graphs.end()) {
    CEM_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
    const hipError_t body = enqueue_plan_body<T>(m, ps, p, batch, m->cap_stream);
    hipGraph_t g = nullptr;
    const hipError_t end = hipStreamEndCapture(m->cap_stream, &g);
    if (body != hipSuccess) { if (g) (void)hipGraphDestroy(g); return hip_status(body, "plan capture"); }
    CEM_TRY(end, "hipStreamEndCapture");
    hipGraphExec_t exec = nullptr;
    const hipError_t inst = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    CEM_TRY(inst, "hipGraphInstantiate");
    it = m->graphs.emplace(key, exec).first;
  }
  CEM_TRY(hipGraphLaunch(it->second, st), "hipGraphLaunch");
  return Status::Ok();
}

}  // namespace

Status rollout(cem_model* m, const float* actions, int n, int horizon, const float* z_obs,
               const float* s0, void* z_pred, hipStream_t st) {
  DeviceGuard guard(m->device);
  hipError_t r = m->bf16 ? enqueue_frame0<bf16>(m, z_obs, 1, m->zobs_t, m->f0, st)
                         : enqueue_frame0<float>(m, z_obs, 1, m->zobs_t, m->f0, st);
  if (r != hipSuccess) return hip_status(r, "frame projection");
  r = m->bf16 ? enqueue_rollout<bf16>(m, actions, n, horizon, s0, m->f0, n, st)
              : enqueue_rollout<float>(m, actions, n, horizon, s0, m->f0, n, st);
  if (r != hipSuccess) return hip_status(r, "rollout kernels");
  const size_t bytes = (size_t)n * m->desc.patches * m->desc.enc_dim * m->esz;
  CEM_TRY(hipMemcpyAsync(z_pred, m->zhat, bytes, hipMemcpyDeviceToDevice, st), "hipMemcpyAsync(z_pred)");
  return Status::Ok();
}

namespace {

// Inputs into the plan state, the rounds (graph replay or direct enqueue), results out.
Status plan_with_state(cem_model* m, const PlanState& ps, bool direct, const cem_params& p, int batch,
                       const float* z_obs, const float* z_goal, const float* s0, float* mu,
                       float* sigma, float* action, int32_t* best_idx, hipStream_t st) {
  const size_t PE = (size_t)m->desc.patches * m->desc.enc_dim, S = m->desc.state_dim;
  const int A = m->desc.action_dim, ha = p.horizon * A, K = p.n_elites;
  const size_t nb = (size_t)batch;
  CEM_TRY(hipMemcpyAsync(ps.zobs, z_obs, nb * PE * 4, hipMemcpyDeviceToDevice, st), "copy z_obs");
  CEM_TRY(hipMemcpyAsync(ps.zgoal, z_goal, nb * PE * 4, hipMemcpyDeviceToDevice, st), "copy z_goal");
  CEM_TRY(hipMemcpyAsync(ps.s0, s0, nb * S * 4, hipMemcpyDeviceToDevice, st), "copy s0");
  CEM_TRY(hipMemcpyAsync(ps.mu_hist, mu, nb * ha * 4, hipMemcpyDeviceToDevice, st), "copy mu");
  CEM_TRY(hipMemcpyAsync(ps.sigma_hist, sigma, nb * ha * 4, hipMemcpyDeviceToDevice, st), "copy sigma");
  CEM_TRY(launch_set_params(ps.params, p.seed, p.plan_id, p.first_round, st), "set params");
  Status s;
  if (direct)
    s = hip_status(m->bf16 ? enqueue_plan_body<bf16>(m, ps, p, batch, st)
                           : enqueue_plan_body<float>(m, ps, p, batch, st), "plan kernels");
  else
    s = m->bf16 ? run_plan<bf16>(m, p, batch, st) : run_plan<float>(m, p, batch, st);
  if (!s.ok()) return s;
  const float* mu_r = ps.mu_hist + (size_t)p.rounds * nb * ha;
  const float* sg_r = ps.sigma_hist + (size_t)p.rounds * nb * ha;
  CEM_TRY(hipMemcpyAsync(mu, mu_r, nb * ha * 4, hipMemcpyDeviceToDevice, st), "copy mu out");
  CEM_TRY(hipMemcpyAsync(sigma, sg_r, nb * ha * 4, hipMemcpyDeviceToDevice, st), "copy sigma out");
  // problem b's action = mu_R[b][0, :], best candidate = its last round's first elite
  CEM_TRY(hipMemcpy2DAsync(action, (size_t)A * 4, mu_r, (size_t)ha * 4, (size_t)A * 4, nb,
                           hipMemcpyDeviceToDevice, st), "copy action");
  if (best_idx)
    CEM_TRY(hipMemcpy2DAsync(best_idx, 4, ps.elites + (size_t)(p.rounds - 1) * nb * K, (size_t)K * 4, 4, nb,
                             hipMemcpyDeviceToDevice, st), "copy best_idx");
  return Status::Ok();
}

}  // namespace

Status plan(cem_model* m, const cem_params& p, int batch, const float* z_obs, const float* z_goal,
            const float* s0, float* mu, float* sigma, float* action, int32_t* best_idx,
            hipStream_t st) {
  DeviceGuard guard(m->device);
  Status s = ensure_plan_state(m, p, batch);
  if (!s.ok()) return s;
  PlanState& ps = m->plan;
  s = plan_with_state(m, ps, false, p, batch, z_obs, z_goal, s0, mu, sigma, action, best_idx, st);
  if (!s.ok()) return s;
  ps.last_n = p.n_samples; ps.last_k = p.n_elites; ps.last_r = p.rounds; ps.last_h = p.horizon;
  ps.last_batch = batch;
  return Status::Ok();
}

Status plan_noalloc(cem_model* m, const cem_params& p, const float* z_obs, const float* z_goal,
                    const float* s0, float* mu, float* sigma, float* action, int32_t* best_idx,
                    hipStream_t st) {
  DeviceGuard guard(m->device);
  Status bad;
  if (m->timers) {
    bad.code = CEM_E_ARG;
    bad.msg = "cem_plan_noalloc: kernel timers are enabled on this model (they record events)";
    return bad;
  }
  const PlanLayout l = plan_layout(m, p.n_samples, p.n_elites, p.rounds, p.horizon * m->desc.action_dim, 1);
  if (l.bytes > kPlanScratchBytes) {
    bad.code = CEM_E_SHAPE;
    bad.msg = "cem_plan_noalloc: the plan state needs " + std::to_string(l.bytes) +
              " bytes, more than the " + std::to_string(kPlanScratchBytes) + "-byte scratch";
    return bad;
  }
  void* base = scratch_of(m->device);
  if (!base) {
    bad.code = CEM_E_INTERNAL;
    bad.msg = "cem_plan_noalloc: no scratch address for this device";
    return bad;
  }
  PlanState ps;
  carve_plan_state(ps, base, l);
  return plan_with_state(m, ps, true, p, 1, z_obs, z_goal, s0, mu, sigma, action, best_idx, st);
}

Status plan_trace(cem_model* m, int kind, void* dst, size_t bytes, hipStream_t st) {
  DeviceGuard guard(m->device);
  const PlanState& ps = m->plan;
  Status bad;
  bad.code = CEM_E_ARG;
  if (!ps.mem || ps.last_r == 0) { bad.msg = "no plan has run on this model"; return bad; }
  const size_t NB = (size_t)ps.last_batch, N = ps.last_n * NB, K = ps.last_k * NB, R = ps.last_r;
  const size_t ha = (size_t)ps.last_h * m->desc.action_dim;
  const void* src = nullptr;
  size_t want = 0;
  switch (kind) {
    case CEM_TRACE_ACTIONS: src = ps.x_hist; want = R * N * ha * 4; break;
    case CEM_TRACE_ENERGY: src = ps.e_hist; want = R * N * 4; break;
    case CEM_TRACE_ELITES: src = ps.elites; want = R * K * 4; break;
    case CEM_TRACE_MU: src = ps.mu_hist; want = (R + 1) * NB * ha * 4; break;
    case CEM_TRACE_SIGMA: src = ps.sigma_hist; want = (R + 1) * NB * ha * 4; break;
    default: bad.msg = "unknown trace kind"; return bad;
  }
  if (bytes != want) {
    bad.code = CEM_E_SHAPE;
    bad.msg = "trace size mismatch: expected " + std::to_string(want) + " bytes";
    return bad;
  }
  CEM_TRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st), "copy trace");
  return Status::Ok();
}

Status timer_read(cem_model* m, int64_t* launches, double* ms, double* flop) {
  DeviceGuard guard(m->device);
  double tot = 0.0, fl = 0.0;
  for (size_t i = 0; i < m->ev_used; ++i) {
    CEM_TRY(hipEventSynchronize(m->ev[i].second), "hipEventSynchronize");
    float t = 0.f;
    CEM_TRY(hipEventElapsedTime(&t, m->ev[i].first, m->ev[i].second), "hipEventElapsedTime");
    tot += t;
    fl += m->ev_flop[i];
  }
  *launches = (int64_t)m->ev_used;
  *ms = tot;
  *flop = fl;
  m->ev_used = 0;
  return Status::Ok();
}

}  // namespace cem
