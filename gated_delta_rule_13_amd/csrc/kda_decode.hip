// Single-token decode step on a resident fp32 state (kda_recurrent_step).
//
// Per chain (sequence, head), following the decay-then-delta form of the page
// "KDA 与 Gated DeltaNet：线性注意力怎样读写有限状态", section 2:
//   S~ = Diag(alpha) S,  p = S~^T k,  d = beta (v - p),  S = S~ + k d^T,  o = S^T q.
// Since S^T q = S~^T q + (k^T q) d, one read of S gives both reductions p and
// y = S~^T q; the state is then updated in registers and written back once. The
// step is a pure HBM stream: 2 * dk * dv * 4 bytes of state traffic per chain
// against about 8 * dk * dv flops.
//
// Layout: one 256-thread workgroup per chain. Thread t owns the float4 column group
// cq = t % (dv / 4) and the rows rg, rg + RG, rg + 2 RG, ... with rg = t / (dv / 4),
// RG = 256 / (dv / 4). A wavefront therefore reads whole 512-byte state rows with
// 16-byte loads. The column reductions over rows go through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;

template <int DK, int DV, typename TIn, bool PER_CHANNEL>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(DecodeArgs a) {
  constexpr int QUADS = DV / 4;
  constexpr int RG = kThreads / QUADS;
  constexpr int RPT = DK / RG;
  static_assert(RPT * RG == DK, "rows must split evenly over row groups");

  __shared__ float s_k[DK];
  __shared__ float s_q[DK];
  __shared__ float s_alpha[DK];
  __shared__ float4 s_red_p[RG][QUADS];
  __shared__ float4 s_red_y[RG][QUADS];
  __shared__ float s_kq[kThreads / 64];

  const int chain = blockIdx.x;  // n * H + h
  const int tid = threadIdx.x;
  const TIn* qp = static_cast<const TIn*>(a.q) + (size_t)chain * DK;
  const TIn* kp = static_cast<const TIn*>(a.k) + (size_t)chain * DK;
  const TIn* vp = static_cast<const TIn*>(a.v) + (size_t)chain * DV;

  // key, query and decay of this token; k^T q by a wavefront reduction
  float kq = 0.f;
  for (int i = tid; i < DK; i += kThreads) {
    const float kk = to_f32(kp[i]);
    const float qq = to_f32(qp[i]);
    s_k[i] = kk;
    s_q[i] = qq;
    s_alpha[i] = __expf(PER_CHANNEL ? a.g[(size_t)chain * DK + i] : a.g[chain]);
    kq += kk * qq;
  }
  for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off, 64);
  if ((tid & 63) == 0) s_kq[tid >> 6] = kq;
  __syncthreads();

  const int cq = tid % QUADS;
  const int rg = tid / QUADS;
  float4* S = reinterpret_cast<float4*>(a.state + (size_t)chain * DK * DV);

  float4 s[RPT];
  float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    float4 x = S[r * QUADS + cq];
    const float al = s_alpha[r];
    x.x *= al; x.y *= al; x.z *= al; x.w *= al;
    s[i] = x;
    const float kr = s_k[r], qr = s_q[r];
    p.x += x.x * kr; p.y += x.y * kr; p.z += x.z * kr; p.w += x.w * kr;
    y.x += x.x * qr; y.y += x.y * qr; y.z += x.z * qr; y.w += x.w * qr;
  }
  s_red_p[rg][cq] = p;
  s_red_y[rg][cq] = y;
  __syncthreads();
  p = make_float4(0.f, 0.f, 0.f, 0.f);
  y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const float4 pp = s_red_p[r][cq], yy = s_red_y[r][cq];
    p.x += pp.x; p.y += pp.y; p.z += pp.z; p.w += pp.w;
    y.x += yy.x; y.y += yy.y; y.z += yy.z; y.w += yy.w;
  }
  float kqs = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) kqs += s_kq[w];

  const float b = a.beta[chain];
  float4 d;
  d.x = b * (to_f32(vp[4 * cq + 0]) - p.x);
  d.y = b * (to_f32(vp[4 * cq + 1]) - p.y);
  d.z = b * (to_f32(vp[4 * cq + 2]) - p.z);
  d.w = b * (to_f32(vp[4 * cq + 3]) - p.w);

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float kr = s_k[r];
    float4 x = s[i];
    x.x += kr * d.x; x.y += kr * d.y; x.z += kr * d.z; x.w += kr * d.w;
    S[r * QUADS + cq] = x;
  }
  if (rg == 0) {
    TIn* op = static_cast<TIn*>(a.o) + (size_t)chain * DV + 4 * cq;
    op[0] = from_f32<TIn>(y.x + kqs * d.x);
    op[1] = from_f32<TIn>(y.y + kqs * d.y);
    op[2] = from_f32<TIn>(y.z + kqs * d.z);
    op[3] = from_f32<TIn>(y.w + kqs * d.w);
  }
}

template <int DK, int DV>
hipError_t launch_dims(const DecodeArgs& a, bool bf16, bool per_channel, hipStream_t stream) {
  const dim3 grid(a.N * a.H), block(kThreads);
  if (bf16) {
    if (per_channel)
      decode_step_kernel<DK, DV, kda::bf16, true><<<grid, block, 0, stream>>>(a);
    else
      decode_step_kernel<DK, DV, kda::bf16, false><<<grid, block, 0, stream>>>(a);
  } else {
    if (per_channel)
      decode_step_kernel<DK, DV, float, true><<<grid, block, 0, stream>>>(a);
    else
      decode_step_kernel<DK, DV, float, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dk, int dv, bool bf16, bool per_channel,
                         hipStream_t stream) {
  if (dk == 128 && dv == 128) return launch_dims<128, 128>(a, bf16, per_channel, stream);
  if (dk == 128 && dv == 64) return launch_dims<128, 64>(a, bf16, per_channel, stream);
  if (dk == 64 && dv == 128) return launch_dims<64, 128>(a, bf16, per_channel, stream);
  if (dk == 64 && dv == 64) return launch_dims<64, 64>(a, bf16, per_channel, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
