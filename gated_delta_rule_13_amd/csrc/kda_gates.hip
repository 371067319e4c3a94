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
// held by d / 8 consecutive lanes, eight channels each, so every bf16 access is one
// 16-byte vector (two for fp32) and the row reductions are d / 8-lane shuffles; a
// wavefront covers 512 / d rows, a thread one row.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr long long kMaxBlocks = 1ll << 24;  // the grid strides beyond this many tiles
constexpr float kEpsL2 = 1e-6f;
constexpr float kGMin = -5.f;  // lower bound of the log-decay

typedef float nf4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;

// Eight consecutive channels of one row: one 16-byte access for bf16, two for fp32.
struct V8 {
  nf4 lo, hi;
};

// NT: a non-temporal load (data read once; measured faster for the epilogue's inputs,
// slower for the prologue's, so each kernel picks).
template <bool NT, typename V>
__device__ __forceinline__ V get(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__device__ __forceinline__ V8 load8(const float* p) {
  return V8{get<NT>(reinterpret_cast<const nf4*>(p)), get<NT>(reinterpret_cast<const nf4*>(p + 4))};
}
template <bool NT>
__device__ __forceinline__ V8 load8(const bf16* p) {
  const bf16x8 v = get<NT>(reinterpret_cast<const bf16x8*>(p));
  return V8{nf4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]},
            nf4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]}};
}

__device__ __forceinline__ void store8(float* p, const V8& x) {
  *reinterpret_cast<nf4*>(p) = x.lo;
  *reinterpret_cast<nf4*>(p + 4) = x.hi;
}
__device__ __forceinline__ void store8(bf16* p, const V8& x) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = static_cast<bf16>(x.lo[i]);
    v[i + 4] = static_cast<bf16>(x.hi[i]);
  }
  *reinterpret_cast<bf16x8*>(p) = v;
}

__device__ __forceinline__ float sumsq(const V8& x) {
  const nf4 a = x.lo * x.lo + x.hi * x.hi;
  return (a[0] + a[1]) + (a[2] + a[3]);
}

__device__ __forceinline__ V8 scale8(const V8& x, float r) { return V8{x.lo * r, x.hi * r}; }

// Sum over the LANES consecutive lanes of a row (LANES a power of two, <= 64).
template <int LANES>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = LANES / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// softplus(x) = max(x, 0) + log1p(e), e = exp(-|x|) in (0, 1], with log1p from the
// identity log1p(e) = 2 atanh(s), s = e / (2 + e) in (0, 1/3], and the atanh series
// s + s^3/3 + ... + s^13/13 (the first omitted term is below 2^-26 of the sum), so the
// result keeps full fp32 relative accuracy also where e is far below 1.
__device__ __forceinline__ float softplus(float x) {
  const float e = __expf(-fabsf(x));
  const float s = e * __builtin_amdgcn_rcpf(2.f + e);
  const float s2 = s * s;
  float p = 1.f / 13.f;
  p = fmaf(p, s2, 1.f / 11.f);
  p = fmaf(p, s2, 1.f / 9.f);
  p = fmaf(p, s2, 1.f / 7.f);
  p = fmaf(p, s2, 1.f / 5.f);
  p = fmaf(p, s2, 1.f / 3.f);
  p = fmaf(p, s2, 1.f);
  return fmaxf(x, 0.f) + 2.f * s * p;
}

// 1 / (1 + exp(-x)); exp(-x) = inf for very negative x gives rcp(inf) = 0.
__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// A block takes a tile of ROWS consecutive tokens of one (sequence, head), so the head
// and its parameters are uniform over the block; the grid covers every tile once (it
// strides only past kMaxBlocks tiles). Rows past the end of the head load its last row
// again (always in bounds) and store nothing.
template <int DK, typename T>
__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueArgs a, int tiles_per_head) {
  constexpr int LANES = DK / 8;
  constexpr int ROWS = kThreads / LANES;
  const int c0 = 8 * (threadIdx.x % LANES);
  const int r0 = threadIdx.x / LANES;
  const long long tiles = (long long)a.B * a.H * tiles_per_head;
  const T* qi = static_cast<const T*>(a.q_in);
  const T* ki = static_cast<const T*>(a.k_in);
  T* qo = static_cast<T*>(a.q_out);
  T* ko = static_cast<T*>(a.k_out);
  for (long long tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const long long bh = tile / tiles_per_head;                 // uniform: scalar unit
    const int t = (int)(tile - bh * tiles_per_head) * ROWS + r0;
    const int h = (int)(bh % a.H);
    const size_t row = (size_t)(bh * a.T + min(t, a.T - 1));
    const size_t off = row * DK + c0;
    const V8 q = load8<false>(qi + off);
    const V8 k = load8<false>(ki + off);
    const V8 u = load8<false>(a.u + off);
    const V8 bias = load8<false>(a.dt_bias + (size_t)h * DK + c0);
    const float bin = a.beta_in ? a.beta_in[row] : 0.f;
    const float sc = -__expf(a.A_log[h]);
    const float rq = rsqrtf(row_sum<LANES>(sumsq(q)) + kEpsL2);
    const float rk = rsqrtf(row_sum<LANES>(sumsq(k)) + kEpsL2);
    V8 g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g.lo[i] = fmaxf(sc * softplus(u.lo[i] + bias.lo[i]), kGMin);
      g.hi[i] = fmaxf(sc * softplus(u.hi[i] + bias.hi[i]), kGMin);
    }
    if (t < a.T) {
      store8(qo + off, scale8(q, rq));
      store8(ko + off, scale8(k, rk));
      store8(a.g_out + off, g);
      if (a.beta_in && c0 == 0) a.beta_out[row] = sigmoid(bin);
    }
  }
}

template <int DV, typename T>
__global__ __launch_bounds__(kThreads) void epilogue_kernel(EpilogueArgs a) {
  constexpr int LANES = DV / 8;
  constexpr int ROWS = kThreads / LANES;
  const int c0 = 8 * (threadIdx.x % LANES);
  const long long rows = (long long)a.B * a.H * a.T;
  const T* oi = static_cast<const T*>(a.o_in);
  const T* zi = static_cast<const T*>(a.z);
  T* oo = static_cast<T*>(a.o_out);
  const V8 w = a.weight ? load8<false>(a.weight + c0)
                        : V8{nf4{1.f, 1.f, 1.f, 1.f}, nf4{1.f, 1.f, 1.f, 1.f}};
  for (long long row = (long long)blockIdx.x * ROWS + threadIdx.x / LANES; row < rows;
       row += (long long)gridDim.x * ROWS) {
    const size_t off = (size_t)row * DV + c0;
    const V8 o = load8<true>(oi + off);
    const V8 z = load8<true>(zi + off);
    const float r = rsqrtf(row_sum<LANES>(sumsq(o)) * (1.f / DV) + a.eps);
    V8 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y.lo[i] = sigmoid(z.lo[i]) * o.lo[i] * r * w.lo[i];
      y.hi[i] = sigmoid(z.hi[i]) * o.hi[i] * r * w.hi[i];
    }
    store8(oo + off, y);
  }
}

unsigned grid_for(long long tiles) {
  return (unsigned)(tiles < kMaxBlocks ? tiles : kMaxBlocks);
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, int dk, bool bf16, hipStream_t stream) {
  const int tile = kThreads / (dk / 8);
  const int tiles_per_head = (a.T + tile - 1) / tile;
  const unsigned grid = grid_for((long long)a.B * a.H * tiles_per_head);
  if (dk == 128) {
    if (bf16) prologue_kernel<128, kda::bf16><<<grid, kThreads, 0, stream>>>(a, tiles_per_head);
    else prologue_kernel<128, float><<<grid, kThreads, 0, stream>>>(a, tiles_per_head);
  } else if (dk == 64) {
    if (bf16) prologue_kernel<64, kda::bf16><<<grid, kThreads, 0, stream>>>(a, tiles_per_head);
    else prologue_kernel<64, float><<<grid, kThreads, 0, stream>>>(a, tiles_per_head);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_epilogue(const EpilogueArgs& a, int dv, bool bf16, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.T;
  const long long tile = kThreads / (dv / 8);
  const unsigned grid = grid_for((rows + tile - 1) / tile);
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
