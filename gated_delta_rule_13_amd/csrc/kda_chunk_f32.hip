// Chunked forward in plain fp32 arithmetic (the kda_chunk_fwd path for float32
// inputs; it also accepts bf16 inputs and is then a slow cross-check path).
//
// The algorithm is the chunkwise form of "Token Mixer I", section "Kimi Delta
// Attention" (WY representation, UT transform, inter-chunk state update and chunk
// output). With G_r the chunk-local inclusive cumulative log-decay (per key channel):
//   A_qk[i,j] = sum_c q_i[c] k_j[c] exp(G_i[c] - G_j[c])          (j <= i)
//   A_kk[i,j] = beta_i sum_c k_i[c] k_j[c] exp(G_i[c] - G_j[c])    (j <  i)
//   Tm = (I + A_kk)^-1                       (forward substitution, column by column)
//   X  = Diag(beta) (V - (K ⊙ e^G) S)        V' = Tm X   (= U - W S of the pages)
//   O  = (Q ⊙ e^G) S + A_qk V'
//   S <- Diag(e^{G_C}) S + (K ⊙ e^{G_C - G})^T V'
// The decay factors of A_qk and A_kk are split at the middle of the chunk, R = G_15:
// e^{G_i - G_j} = e^{G_i - R} e^{R - G_j}. Over 32 tokens with g >= -5 each factor lies in
// [e^-80, e^80], inside the fp32 range, and their product is the exact weighting, so the
// tiles are plain dot products of q e^{G - R} and k e^{R - G}; nothing is divided by a decay,
// and every other exponent is G itself or G_C - G, at most 1.
//
// Gated Delta Rule-2 ("Token Mixer I", section "Gated DeltaNet-2"): the read side uses
// the erase-gated keys B * K in place of Diag(beta) K (in A_kk and in the prediction), and
// the values are gated per channel, X = W * V - ((B * K) e^G) S; the rest is unchanged.
//
// One 256-thread workgroup per (chain, block of DVB value columns): value columns are
// independent (the decay acts on the rows of S), so the state pass splits over them.
// Chunk size 32 keeps the fp32 tiles of q, k and G in LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kC = 32;    // chunk length of this path
constexpr int kDVB = 32;  // value columns per workgroup

template <int DK, typename TIn, bool PER_CHANNEL, bool GDR2>
__global__ __launch_bounds__(kThreads) void chunk_f32_kernel(ChunkArgs a, int n_dvb) {
  __shared__ float sQ[kC][DK];
  __shared__ float sK[kC][DK];
  __shared__ float sG[kC][DK];   // cumulative log-decay, later K ⊙ e^{G_C - G}
  __shared__ float sQr[kC][DK + 1];  // q e^{G - R}, then (B *) k e^{G - R}
  __shared__ float sKd[kC][DK + 1];  // k e^{R - G}
  __shared__ float sAqk[kC][kC + 1];
  __shared__ float sAkk[kC][kC + 1];
  __shared__ float sTm[kC][kC + 1];
  __shared__ float sV[kC][kDVB];  // V, later V'
  __shared__ float sX[kC][kDVB];
  __shared__ float sS[DK][kDVB];
  __shared__ float sBeta[kC];
  __shared__ float sGC[DK];
  // Gated Delta Rule-2: erase-gated keys b * k (the read side) and the write gates
  __shared__ float sE[GDR2 ? kC : 1][GDR2 ? DK : 1];
  __shared__ float sW[GDR2 ? kC : 1][GDR2 ? kDVB : 1];

  const int tid = threadIdx.x;
  const int chain = blockIdx.x / n_dvb;
  const int dvb = blockIdx.x % n_dvb;
  const int n = chain / a.H;
  const int h = chain % a.H;
  const int DV = a.dv;
  const TokenRange tr = token_range(a.cu, n, a.T);
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0;  // row of the first token
  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
  const TIn* v = static_cast<const TIn*>(a.v);
  TIn* o = static_cast<TIn*>(a.o);
  const int col0 = dvb * kDVB;
  const size_t state_off = ((size_t)n * a.H + h) * DK * DV;

  for (int idx = tid; idx < DK * kDVB; idx += kThreads) {
    const int c = idx / kDVB, j = idx % kDVB;
    sS[c][j] = a.s0 ? a.s0[state_off + (size_t)c * DV + col0 + j] : 0.f;
  }

  for (int c0 = 0; c0 < tr.len; c0 += kC) {
    const int nt = min(kC, tr.len - c0);
    __syncthreads();  // previous chunk finished with every LDS tile
    // -- load the chunk; positions past the sequence end are identity tokens
    for (int idx = tid; idx < kC * DK; idx += kThreads) {
      const int t = idx / DK, c = idx % DK;
      const bool ok = t < nt;
      const size_t r = row0 + c0 + t;
      sQ[t][c] = ok ? to_f32(q[r * DK + c]) : 0.f;
      sK[t][c] = ok ? to_f32(k[r * DK + c]) : 0.f;
      sG[t][c] = ok ? (PER_CHANNEL ? a.g[r * DK + c] : a.g[r]) : 0.f;
      if (GDR2) sE[t][c] = ok ? a.erase[r * DK + c] * sK[t][c] : 0.f;
    }
    for (int idx = tid; idx < kC * kDVB; idx += kThreads) {
      const int t = idx / kDVB, j = idx % kDVB;
      sV[t][j] = t < nt ? to_f32(v[(row0 + c0 + t) * DV + col0 + j]) : 0.f;
      if (GDR2) sW[t][j] = t < nt ? a.write[(row0 + c0 + t) * DV + col0 + j] : 0.f;
    }
    if (tid < kC) sBeta[tid] = tid < nt ? (GDR2 ? 1.f : a.beta[row0 + c0 + tid]) : 0.f;
    __syncthreads();
    // -- chunk-local inclusive cumulative log-decay
    for (int c = tid; c < DK; c += kThreads) {
      float run = 0.f;
      for (int t = 0; t < kC; ++t) {
        run += sG[t][c];
        sG[t][c] = run;
      }
      sGC[c] = run;
    }
    __syncthreads();
    // -- the factors of the decay split at R = G_15 (q, k e^{G - R} and k e^{R - G})
    for (int idx = tid; idx < kC * DK; idx += kThreads) {
      const int t = idx / DK, c = idx % DK;
      const float d = sG[t][c] - sG[kC / 2 - 1][c];
      sQr[t][c] = sQ[t][c] * __expf(d);
      sKd[t][c] = sK[t][c] * __expf(-d);
    }
    __syncthreads();
    // -- A_qk (inclusive lower) and A_kk (strict lower, rows scaled by beta); the read-side
    // key of A_kk, (B *) k e^{G - R}, is formed in place of q after A_qk
    for (int pidx = tid; pidx < kC * kC; pidx += kThreads) {
      const int i = pidx / kC, j = pidx % kC;
      float aq = 0.f;
      if (j <= i)
        for (int c = 0; c < DK; ++c) aq += sQr[i][c] * sKd[j][c];
      sAqk[i][j] = aq;
    }
    __syncthreads();
    for (int idx = tid; idx < kC * DK; idx += kThreads) {
      const int t = idx / DK, c = idx % DK;
      sQr[t][c] = (GDR2 ? sE[t][c] : sK[t][c]) * __expf(sG[t][c] - sG[kC / 2 - 1][c]);
    }
    __syncthreads();
    for (int pidx = tid; pidx < kC * kC; pidx += kThreads) {
      const int i = pidx / kC, j = pidx % kC;
      float ak = 0.f;
      if (j < i)
        for (int c = 0; c < DK; ++c) ak += sQr[i][c] * sKd[j][c];
      sAkk[i][j] = j < i ? sBeta[i] * ak : 0.f;
    }
    __syncthreads();
    // -- Tm = (I + A_kk)^-1 by forward substitution, one column per thread, the column in
    // registers (row i of column j is -sum_{m < i} A_kk[i][m] Tm[m][j]; Tm[m][j] = 0 for
    // m < j and 1 at m = j)
    if (tid < kC) {
      const int j = tid;
      float tcol[kC];
#pragma unroll
      for (int i = 0; i < kC; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc += sAkk[i][m] * tcol[m];
        tcol[i] = i < j ? 0.f : (i == j ? 1.f : -acc);
      }
#pragma unroll
      for (int i = 0; i < kC; ++i) sTm[i][j] = tcol[i];
    }
    // -- decayed operands, in place: Q <- Q e^G, K <- K e^G, G <- K e^{G_C - G}
    for (int idx = tid; idx < kC * DK; idx += kThreads) {
      const int t = idx / DK, c = idx % DK;
      const float G = sG[t][c];
      const float e = __expf(G);
      const float kk = sK[t][c];
      sG[t][c] = kk * __expf(sGC[c] - G);
      sQ[t][c] *= e;
      sK[t][c] = kk * e;
      if (GDR2) sE[t][c] *= e;
    }
    __syncthreads();
    // -- X = Diag(beta) (V - (K e^G) S); Gated Delta Rule-2: X = W * V - ((B * K) e^G) S
    for (int idx = tid; idx < kC * kDVB; idx += kThreads) {
      const int t = idx / kDVB, j = idx % kDVB;
      if (GDR2) {
        float acc = sW[t][j] * sV[t][j];
        for (int c = 0; c < DK; ++c) acc -= sE[t][c] * sS[c][j];
        sX[t][j] = acc;
      } else {
        float acc = sV[t][j];
        for (int c = 0; c < DK; ++c) acc -= sK[t][c] * sS[c][j];
        sX[t][j] = sBeta[t] * acc;
      }
    }
    __syncthreads();
    // -- V' = Tm X
    for (int idx = tid; idx < kC * kDVB; idx += kThreads) {
      const int t = idx / kDVB, j = idx % kDVB;
      float acc = 0.f;
      for (int m = 0; m <= t; ++m) acc += sTm[t][m] * sX[m][j];
      sV[t][j] = acc;
    }
    __syncthreads();
    // -- O = (Q e^G) S + A_qk V'
    for (int idx = tid; idx < kC * kDVB; idx += kThreads) {
      const int t = idx / kDVB, j = idx % kDVB;
      if (t < nt) {
        float acc = 0.f;
        for (int c = 0; c < DK; ++c) acc += sQ[t][c] * sS[c][j];
        for (int m = 0; m <= t; ++m) acc += sAqk[t][m] * sV[m][j];
        o[(row0 + c0 + t) * DV + col0 + j] = from_f32<TIn>(acc);
      }
    }
    __syncthreads();
    // -- S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T V'
    for (int idx = tid; idx < DK * kDVB; idx += kThreads) {
      const int c = idx / kDVB, j = idx % kDVB;
      float acc = __expf(sGC[c]) * sS[c][j];
      for (int t = 0; t < kC; ++t) acc += sG[t][c] * sV[t][j];
      sS[c][j] = acc;
    }
  }
  __syncthreads();
  if (a.sT) {
    for (int idx = tid; idx < DK * kDVB; idx += kThreads) {
      const int c = idx / kDVB, j = idx % kDVB;
      a.sT[state_off + (size_t)c * DV + col0 + j] = sS[c][j];
    }
  }
}

template <int DK, typename TIn, bool PER_CHANNEL>
void launch_gates(const ChunkArgs& a, dim3 grid, int n_dvb, hipStream_t stream) {
  if (a.erase)
    chunk_f32_kernel<DK, TIn, PER_CHANNEL, true><<<grid, dim3(kThreads), 0, stream>>>(a, n_dvb);
  else
    chunk_f32_kernel<DK, TIn, PER_CHANNEL, false><<<grid, dim3(kThreads), 0, stream>>>(a, n_dvb);
}

template <int DK>
hipError_t launch_dk(const ChunkArgs& a, bool bf16, bool per_channel, hipStream_t stream) {
  const int n_dvb = a.dv / kDVB;
  const dim3 grid(a.N * a.H * n_dvb);
  if (bf16) {
    if (per_channel) launch_gates<DK, kda::bf16, true>(a, grid, n_dvb, stream);
    else launch_gates<DK, kda::bf16, false>(a, grid, n_dvb, stream);
  } else {
    if (per_channel) launch_gates<DK, float, true>(a, grid, n_dvb, stream);
    else launch_gates<DK, float, false>(a, grid, n_dvb, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_f32(const ChunkArgs& a, bool bf16, bool per_channel, hipStream_t stream) {
  if (a.dv % kDVB != 0) return hipErrorInvalidValue;
  if (a.dk == 128) return launch_dk<128>(a, bf16, per_channel, stream);
  if (a.dk == 64) return launch_dk<64>(a, bf16, per_channel, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
