// The steps on either side of the operator, each fused into one streaming pass.
//
// Prologue ("Token Mixer I", section "The Kimi Linear Model Architecture", neural
// parameterization; the decay function of the page "阅读笔记: Kimi Delta Attention",
// section 6): per head and token,
//   q, k <- L2Norm(q, k) = x / sqrt(sum x^2 + 1e-6) over the key channels,
//   g    <- max(-exp(A_log[h]) * softplus(u + dt_bias[h, :]), -5)   (fp32 log-decay, with
//           KDA's lower bound g_min = -5 from the knowledge map of the page
//           "【轻量化复刻大模型】线性注意力（Linear Attention）", section 3.1),
//   beta <- Sigmoid(beta pre-activation).
// Epilogue: o <- Sigmoid(z) * o / sqrt(mean o^2 + eps) * w over the value channels (the
// per-head RMSNorm and output gate before the output projection).
//
// Both are pure HBM streams (every byte read once, written once). A row of d channels is
// held by d / 4 consecutive lanes, four channels each, so loads and stores are 8- or
// 16-byte vectors and the row reductions are d / 4-lane shuffles; a wavefront covers
// 256 / d rows at a time and the grid strides over all rows.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 4096;
constexpr float kEpsL2 = 1e-6f;
constexpr float kGMin = -5.f;  // lower bound of the log-decay

typedef float nf4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

template <typename T>
__device__ __forceinline__ nf4 load4(const T* p);
template <>
__device__ __forceinline__ nf4 load4<float>(const float* p) {
  return *reinterpret_cast<const nf4*>(p);
}
template <>
__device__ __forceinline__ nf4 load4<bf16>(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return nf4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
             static_cast<float>(v[3])};
}

template <typename T>
__device__ __forceinline__ void store4(T* p, nf4 x);
template <>
__device__ __forceinline__ void store4<float>(float* p, nf4 x) {
  *reinterpret_cast<nf4*>(p) = x;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, nf4 x) {
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = static_cast<bf16>(x[i]);
  *reinterpret_cast<bf16x4*>(p) = v;
}

// Sum over the LANES consecutive lanes of a row (LANES a power of two, <= 64).
template <int LANES>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = LANES / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float softplus(float x) {
  return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

template <int DK, typename T>
__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueArgs a) {
  constexpr int LANES = DK / 4;
  constexpr int ROWS = kThreads / LANES;  // rows per block and pass
  const int lane_in_row = threadIdx.x % LANES;
  const long long rows = (long long)a.B * a.H * a.T;
  const T* qi = static_cast<const T*>(a.q_in);
  const T* ki = static_cast<const T*>(a.k_in);
  T* qo = static_cast<T*>(a.q_out);
  T* ko = static_cast<T*>(a.k_out);
  for (long long row = (long long)blockIdx.x * ROWS + threadIdx.x / LANES; row < rows;
       row += (long long)gridDim.x * ROWS) {
    const int h = (int)((row / a.T) % a.H);
    const size_t off = (size_t)row * DK + 4 * lane_in_row;
    const nf4 q = load4<T>(qi + off);
    const nf4 k = load4<T>(ki + off);
    const nf4 u = load4<float>(a.u + off);
    const nf4 bias = load4<float>(a.dt_bias + (size_t)h * DK + 4 * lane_in_row);
    const float sq = row_sum<LANES>(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
    const float sk = row_sum<LANES>(k[0] * k[0] + k[1] * k[1] + k[2] * k[2] + k[3] * k[3]);
    const float rq = 1.f / sqrtf(sq + kEpsL2), rk = 1.f / sqrtf(sk + kEpsL2);
    const float scale = -__expf(a.A_log[h]);
    nf4 g;
#pragma unroll
    for (int i = 0; i < 4; ++i) g[i] = fmaxf(scale * softplus(u[i] + bias[i]), kGMin);
    store4<T>(qo + off, q * rq);
    store4<T>(ko + off, k * rk);
    store4<float>(a.g_out + off, g);
    if (a.beta_in && lane_in_row == 0) a.beta_out[row] = sigmoid(a.beta_in[row]);
  }
}

template <int DV, typename T>
__global__ __launch_bounds__(kThreads) void epilogue_kernel(EpilogueArgs a) {
  constexpr int LANES = DV / 4;
  constexpr int ROWS = kThreads / LANES;
  const int lane_in_row = threadIdx.x % LANES;
  const long long rows = (long long)a.B * a.H * a.T;
  const T* oi = static_cast<const T*>(a.o_in);
  const T* zi = static_cast<const T*>(a.z);
  T* oo = static_cast<T*>(a.o_out);
  const nf4 w = a.weight ? load4<float>(a.weight + 4 * lane_in_row) : nf4{1.f, 1.f, 1.f, 1.f};
  for (long long row = (long long)blockIdx.x * ROWS + threadIdx.x / LANES; row < rows;
       row += (long long)gridDim.x * ROWS) {
    const size_t off = (size_t)row * DV + 4 * lane_in_row;
    const nf4 o = load4<T>(oi + off);
    const nf4 z = load4<T>(zi + off);
    const float ss = row_sum<LANES>(o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3]);
    const float r = 1.f / sqrtf(ss * (1.f / DV) + a.eps);
    nf4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = sigmoid(z[i]) * o[i] * r * w[i];
    store4<T>(oo + off, y);
  }
}

unsigned grid_for(long long rows, int rows_per_block) {
  const long long blocks = (rows + rows_per_block - 1) / rows_per_block;
  return (unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks);
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, int dk, bool bf16, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.T;
  const unsigned grid = grid_for(rows, kThreads / (dk / 4));
  if (dk == 128) {
    if (bf16) prologue_kernel<128, kda::bf16><<<grid, kThreads, 0, stream>>>(a);
    else prologue_kernel<128, float><<<grid, kThreads, 0, stream>>>(a);
  } else if (dk == 64) {
    if (bf16) prologue_kernel<64, kda::bf16><<<grid, kThreads, 0, stream>>>(a);
    else prologue_kernel<64, float><<<grid, kThreads, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_epilogue(const EpilogueArgs& a, int dv, bool bf16, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.T;
  const unsigned grid = grid_for(rows, kThreads / (dv / 4));
  if (dv == 128) {
    if (bf16) epilogue_kernel<128, kda::bf16><<<grid, kThreads, 0, stream>>>(a);
    else epilogue_kernel<128, float><<<grid, kThreads, 0, stream>>>(a);
  } else if (dv == 64) {
    if (bf16) epilogue_kernel<64, kda::bf16><<<grid, kThreads, 0, stream>>>(a);
    else epilogue_kernel<64, float><<<grid, kThreads, 0, stream>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kda
