// Token embedding of one frame block.
//
// Page "Real-Time Inference for JEPA World Model Architectures with Ray",
// section 01: each candidate action sequence is pushed through the
// action-conditioned predictor together with the encoded frame and the joint
// state (section 02: a camera frame plus joint state is the robot's input).
// Block layout per candidate n at step t (B = P + 2 rows of x):
//   row n*B + 0      action token  a_t W_a + b_a
//   row n*B + 1      state token   s_t W_s + b_s,  s_t = s_0 + a_0 + ... + a_{t-1}
//   rows n*B + 2 + p frame tokens  f_t W_in + b_in  (f_0 = z_obs for every n)
// The frame rows of step 0 are identical for all candidates: the projection
// f_0 W_in + b_in is computed once per plan and broadcast here.  Later steps'
// frame rows are written by the in-projection GEMM's epilogue.
// All of this is bandwidth work: the broadcast writes N*P*d values.
#include "kernels.hpp"

namespace cem {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ in,
                                                      T* __restrict__ out, long long count) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) out[i] = Elem<T>::from_f32(in[i]);
}

// grid: N blocks; each block writes the action and state rows of one candidate.
template <typename T>
__global__ __launch_bounds__(256) void embed_action_state_kernel(
    const float* __restrict__ X, int H, int t, int A, int S, const float* __restrict__ s0,
    const float* __restrict__ wa, const float* __restrict__ ba, const float* __restrict__ ws,
    const float* __restrict__ bs, T* __restrict__ x, int B, int d, int n_per) {
  __shared__ float act[32];
  __shared__ float st[32];
  const int n = blockIdx.x;
  s0 += (long long)(n / n_per) * S;   // this candidate's problem
  const float* xn = X + (long long)n * H * A;
  if (threadIdx.x < A) act[threadIdx.x] = xn[t * A + threadIdx.x];
  if (threadIdx.x < S) {
    // the state advances by each executed action delta: s_t = s_0 + sum_{tau<t} a_tau
    float s = s0[threadIdx.x];
    for (int tau = 0; tau < t; ++tau) s = s + (threadIdx.x < A ? xn[tau * A + threadIdx.x] : 0.f);
    st[threadIdx.x] = s;
  }
  __syncthreads();
  T* ra = x + (long long)n * B * d;
  T* rs = ra + d;
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    float va = ba[j], vs = bs[j];
    for (int i = 0; i < A; ++i) va += act[i] * wa[(long long)i * d + j];
    for (int i = 0; i < S; ++i) vs += st[i] * ws[(long long)i * d + j];
    ra[j] = Elem<T>::from_f32(va);
    rs[j] = Elem<T>::from_f32(vs);
  }
}

// grid: (ceil(P*d/8 / 256), N); 16-byte copies when rows are 16-byte multiples.
template <typename T>
__global__ __launch_bounds__(256) void broadcast_frame_kernel(const T* __restrict__ f0, int P,
                                                              int d, T* __restrict__ x, int B,
                                                              int n_per) {
  constexpr int V = 16 / sizeof(T);
  const int n = blockIdx.y;
  f0 += (long long)(n / n_per) * P * d;   // this candidate's problem
  const long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (i >= (long long)P * d) return;
  const int p = (int)(i / d), j = (int)(i % d);
  T* dst = x + ((long long)n * B + 2 + p) * d + j;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(f0 + i);
}

// Layer 0 of the first frame block: the rows every candidate of a problem shares and the
// candidates' own action rows, packed into one compact block (16 bytes a thread).
__global__ __launch_bounds__(256) void gather_layer0_kernel(const bf16* __restrict__ x, int B, int d,
                                                            int problems, int n_per, long long count,
                                                            bf16* __restrict__ xc) {
  const long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= count) return;
  const int r = (int)(i / d), j = (int)(i % d);
  const int shared = problems * (B - 1);
  const long long src = r < shared ? (long long)(r / (B - 1)) * n_per * B + 1 + r % (B - 1)
                                   : (long long)(r - shared) * B;
  *reinterpret_cast<uint4*>(xc + i) = *reinterpret_cast<const uint4*>(x + src * d + j);
}

}  // namespace

hipError_t launch_gather_layer0(const bf16* x, int B, int d, int problems, int n_per, int N,
                                bf16* xc, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  if (problems <= 0 || n_per <= 0 || N != problems * n_per || B < 2 || d <= 0 || d % 8 != 0)
    return hipErrorInvalidValue;
  const long long count = ((long long)problems * (B - 1) + N) * d;
  gather_layer0_kernel<<<(unsigned)((count / 8 + 255) / 256), 256, 0, stream>>>(x, B, d, problems,
                                                                              n_per, count, xc);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_convert(const float* in, T* out, long long count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  convert_kernel<T><<<(unsigned)((count + 255) / 256), 256, 0, stream>>>(in, out, count);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_embed_action_state(const float* X, int N, int H, int t, int A, int S,
                                     const float* s0, const float* wa, const float* ba,
                                     const float* ws, const float* bs, T* x, int B, int d,
                                     int n_per, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  if (n_per <= 0) return hipErrorInvalidValue;
  embed_action_state_kernel<T><<<N, 256, 0, stream>>>(X, H, t, A, S, s0, wa, ba, ws, bs, x, B, d,
                                                      n_per);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_broadcast_frame(const T* f0, int P, int d, T* x, int N, int B, int n_per,
                                  hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  if (n_per <= 0) return hipErrorInvalidValue;
  constexpr int V = 16 / sizeof(T);
  const long long vec = (long long)P * d / V;   // d % 64 == 0, so rows are whole vectors
  dim3 grid((unsigned)((vec + 255) / 256), (unsigned)N);
  broadcast_frame_kernel<T><<<grid, 256, 0, stream>>>(f0, P, d, x, B, n_per);
  return hipGetLastError();
}

#define INST(T)                                                                                  \
  template hipError_t launch_convert<T>(const float*, T*, long long, hipStream_t);              \
  template hipError_t launch_embed_action_state<T>(const float*, int, int, int, int, int,       \
                                                   const float*, const float*, const float*,    \
                                                   const float*, const float*, T*, int, int,    \
                                                   int, hipStream_t);                           \
  template hipError_t launch_broadcast_frame<T>(const T*, int, int, T*, int, int, int,          \
                                                hipStream_t);
INST(float)
INST(bf16)
#undef INST

}  // namespace cem
