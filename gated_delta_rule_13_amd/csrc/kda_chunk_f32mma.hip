// Chunked forward on the fp32 matrix cores (16x16x4 fp32 products): the kda_chunk_fwd path
// for float32 inputs, for dk = 64, and for whatever the bf16 kernel does not take (dv = 64
// chains past 2^22 tokens, long axes without a workspace). Every operand and every product is
// fp32; bf16 inputs are widened on load and the outputs rounded on store.
//
// The algorithm is the chunkwise form of "Token Mixer I", section "Kimi Delta Attention"
// (WY representation, UT transform, inter-chunk state update, chunk output), taken over
// blocks of 16 tokens. With G_t the block-local inclusive cumulative log decay per key
// channel and R = G_7:
//   A_qk[i][j] = sum_c q_i[c] k_j[c] e^{G_i[c] - G_j[c]}           (j <= i)
//   A_kk[i][j] = sum_c k_i[c] k_j[c] e^{G_i[c] - G_j[c]}           (j <  i)
//   Tm = (I + Diag(beta) A_kk)^-1,   V' = Tm Diag(beta) (V - (K e^G) S)
//   O  = (Q e^G) S + A_qk V',        S <- Diag(e^{G_15}) S + (K e^{G_15 - G})^T V'
// The decay weights of A_qk and A_kk are split at the block's middle,
// e^{G_i - G_j} = e^{G_i - R} e^{R - G_j}; with g >= -5 each factor lies in [e^-40, e^40]
// and every other factor in [e^-80, 1], all inside the fp32 range, so nothing is divided by
// a decay. Tm is the exact nilpotent product (I - N)(I + N^2)(I + N^4)(I + N^8) on the
// matrix cores.
//
// Gated Delta Rule-2 ("Token Mixer I", section "Gated DeltaNet-2"): the read side takes the
// erase-gated keys b * k in A_kk and in the prediction, beta is 1, and the values are the
// write-gated w * V.
//
// One 256-thread workgroup per (chain, 64 value columns); wavefront w owns value columns
// 16 w .. 16 w + 15 of the workgroup's and their dk x 16 slice of S in accumulator registers.
// Per block: the inputs (prefetched into registers during the previous block) go to LDS,
// the cumulative decay and the decayed factors are formed there, wavefront 0 forms A_qk and
// wavefront 1 A_kk and Tm while every wavefront forms its (K e^G) S and (Q e^G) S; then
// V', the outputs and the state update. Plain 64-bit addressing: any T.
//
// Operand layouts of the 16x16x4 product D[i][j] += sum_k A[i][k] B[k][j]: lane 16 p + r
// gives A[r][p] and B[p][r] and holds D[4 p + e][r]. A state tile S[16 m + 4 p + e][col r]
// held as element e is directly the B operand of the product whose contraction index p
// stands for channel 16 m + 4 p + e, and likewise every accumulator tile of 16 tokens is
// the B operand of a contraction over those tokens; the A operands are then read from LDS
// rows at the same channels (or tokens).
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kB = 16;            // tokens per block
constexpr int kCols = 64;         // value columns per workgroup (16 per wavefront)

template <int DK, bool GDR2>
struct F32Smem {
  float q[kB][DK];                // raw block inputs (fp32)
  float k[kB][DK];
  float g[kB][DK];                // log decay, then its cumulative sum G
  float er[GDR2 ? kB : 1][GDR2 ? DK : 1];  // erase gates (Gated Delta Rule-2)
  float v[kB][kCols + 1];         // V, or w * V, of the workgroup's columns
  float beta[kB];
  // (read as 16-byte vectors: aligned)
  alignas(16) float qP[kB][DK + 4];   // q e^G
  alignas(16) float kP[kB][DK + 4];   // (b *) k e^G
  alignas(16) float qh[kB][DK + 4];   // q e^{G - R}
  alignas(16) float kh[kB][DK + 4];   // (b *) k e^{G - R}
  alignas(16) float kb[kB][DK + 4];   // k e^{R - G}
  float kE[kB][DK + 1];               // k e^{G_15 - G}
  alignas(16) float tot[DK];          // e^{G_15}
  alignas(16) float aqk[kB][kB + 4];  // A_qk (lower, diagonal included)
  alignas(16) float tm[kB][kB + 4];   // Tm
  float nn[kB][kB + 1];               // Diag(beta) A_kk (strictly lower), for its transpose
};

// Registers of one block's inputs for this thread: elements [8 tid, 8 tid + 8) of the
// block's q, k, g (and erase) rows, elements [4 tid, 4 tid + 4) of its value columns.
template <int DK, bool GDR2>
struct F32Regs {
  float q[8], k[8], g[8], e[GDR2 ? 8 : 1], v[4], w[GDR2 ? 4 : 1];
  float beta;
};

template <int DK, typename TIn, bool PER_CHANNEL, bool GDR2>
__device__ __forceinline__ void load_f32_block(F32Regs<DK, GDR2>& r, const ChunkArgs& a,
                                               size_t row, int nt, int col0, int tid) {
  constexpr int kPer = kB * DK / kThreads;  // 8 (dk = 128) or 4 (dk = 64)
  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
  const TIn* v = static_cast<const TIn*>(a.v);
  const int idx = kPer * tid, t = idx / DK, c = idx % DK;
  const bool ok = t < nt;
  const size_t off = (row + t) * DK + c;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool in = ok && i < kPer;
    r.q[i] = in ? to_f32(q[off + i]) : 0.f;
    r.k[i] = in ? to_f32(k[off + i]) : 0.f;
    r.g[i] = in ? (PER_CHANNEL ? a.g[off + i] : a.g[row + t]) : 0.f;
    if constexpr (GDR2) r.e[i] = in ? a.erase[off + i] : 0.f;
  }
  const int tv = tid / 16, cv = 4 * (tid % 16);
  const bool okv = tv < nt;
  const size_t offv = (row + tv) * a.dv + col0 + cv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[i] = okv ? to_f32(v[offv + i]) : 0.f;
    if constexpr (GDR2) r.w[i] = okv ? a.write[offv + i] : 0.f;
  }
  r.beta = (!GDR2 && tid < nt) ? a.beta[row + tid] : 0.f;
}

template <int DK, bool GDR2>
__device__ __forceinline__ void store_f32_block(F32Smem<DK, GDR2>& sm, const F32Regs<DK, GDR2>& r,
                                                int tid) {
  constexpr int kPer = kB * DK / kThreads;
  const int idx = kPer * tid, t = idx / DK, c = idx % DK;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    sm.q[t][c + i] = r.q[i];
    sm.k[t][c + i] = r.k[i];
    sm.g[t][c + i] = r.g[i];
    if constexpr (GDR2) sm.er[t][c + i] = r.e[i];
  }
  const int tv = tid / 16, cv = 4 * (tid % 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.v[tv][cv + i] = GDR2 ? r.w[i] * r.v[i] : r.v[i];
  if (tid < kB) sm.beta[tid] = GDR2 ? 1.f : r.beta;
}

// Row operand of lane (r, p) for the 16x16x4 products over channels 16 m + 4 p + e: the
// four channels of row r as one vector.
template <int LD>
__device__ __forceinline__ f32x4 row4(const float (*x)[LD], int r, int c) {
  return *reinterpret_cast<const f32x4*>(&x[r][c]);
}

template <int DK, typename TIn, bool PER_CHANNEL, bool GDR2>
__global__ __launch_bounds__(kThreads) void chunk_f32mma_kernel(ChunkArgs a, int groups) {
  constexpr int NM = DK / 16;       // row tiles of S
  __shared__ __align__(16) F32Smem<DK, GDR2> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rr = lane & 15, p = lane >> 4;
  const int chain = blockIdx.x / groups, grp = blockIdx.x % groups;
  const int n = chain / a.H, h = chain % a.H;
  const int DV = a.dv;
  const int col0 = grp * kCols;           // the workgroup's first value column
  const int col = col0 + 16 * wave + rr;  // this lane's value column
  const TokenRange tr = token_range(a.cu, n, a.T);
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0;
  const size_t mat = ((size_t)n * a.H + h) * DK * DV;

  // S_acc[m][e] = S[16 m + 4 p + e][col]
  f32x4 S_acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S_acc[m][e] = a.s0 ? a.s0[mat + (size_t)(16 * m + 4 * p + e) * DV + col] : 0.f;

  F32Regs<DK, GDR2> regs;
  const int nblk = (tr.len + kB - 1) / kB;
  if (nblk > 0) load_f32_block<DK, TIn, PER_CHANNEL, GDR2>(regs, a, row0, tr.len, col0, tid);
  for (int b = 0; b < nblk; ++b) {
    const int nt = min(kB, tr.len - kB * b);  // tokens of this block (later ones: identity)
    // 1. the block's inputs to LDS (every wavefront has finished the previous block: the
    // barrier after this step orders the overwrite of the factors below)
    store_f32_block<DK, GDR2>(sm, regs, tid);
    __syncthreads();
    // 2. cumulative log decay per channel
    if (tid < DK) {
      float run = 0.f;
#pragma unroll
      for (int t = 0; t < kB; ++t) {
        run += sm.g[t][tid];
        sm.g[t][tid] = run;
      }
      sm.tot[tid] = __expf(run);
    }
    __syncthreads();
    // 3. the decayed factors (identity tokens have q = k = 0 and g = 0)
    for (int idx = tid; idx < kB * DK; idx += kThreads) {
      const int t = idx / DK, c = idx % DK;
      const float G = sm.g[t][c], R = sm.g[kB / 2 - 1][c], GC = sm.g[kB - 1][c];
      const float eR = __expf(G - R);
      const float qf = sm.q[t][c], kf = sm.k[t][c];
      const float kr = GDR2 ? sm.er[t][c] * kf : kf;  // the read-side key
      const float eG = __expf(G);
      sm.qP[t][c] = qf * eG;
      sm.kP[t][c] = kr * eG;
      sm.qh[t][c] = qf * eR;
      sm.kh[t][c] = kr * eR;
      sm.kb[t][c] = kf * __expf(R - G);
      sm.kE[t][c] = kf * __expf(GC - G);
    }
    __syncthreads();
    // the next block's inputs, in flight during the products below
    if (b + 1 < nblk)
      load_f32_block<DK, TIn, PER_CHANNEL, GDR2>(regs, a, row0 + kB * (b + 1),
                                                 tr.len - kB * (b + 1), col0, tid);
    // 4. wavefront 0: A_qk; wavefront 1: A_kk and Tm (LDS)
    if (wave == 0) {
      f32x4 acc = zero4();
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const f32x4 x = row4<DK + 4>(sm.qh, rr, 16 * m + 4 * p);
        const f32x4 y = row4<DK + 4>(sm.kb, rr, 16 * m + 4 * p);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(x[e], y[e], acc);
      }
      // acc[e] = A_qk[4 p + e][rr]
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.aqk[4 * p + e][rr] = rr <= 4 * p + e ? acc[e] : 0.f;
    } else if (wave == 1) {
      f32x4 acc = zero4();
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const f32x4 x = row4<DK + 4>(sm.kh, rr, 16 * m + 4 * p);
        const f32x4 y = row4<DK + 4>(sm.kb, rr, 16 * m + 4 * p);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(x[e], y[e], acc);
      }
      f32x4 nc, nr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * p + e;
        nc[e] = rr < i ? sm.beta[i] * acc[e] : 0.f;  // N[i][rr]
        sm.nn[i][rr] = nc[e];
      }
      wave_lds_fence();
#pragma unroll
      for (int e = 0; e < 4; ++e) nr[e] = sm.nn[rr][4 * p + e];  // N[rr][4 p + e]
      const f32x4 inv = unit_lower_inverse(nc, nr, rr, p);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.tm[4 * p + e][rr] = inv[e];
    }
    // every wavefront: X = ((b *) K e^G) S and (Q e^G) S for its columns
    f32x4 X = zero4(), O = zero4();
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const f32x4 xk = row4<DK + 4>(sm.kP, rr, 16 * m + 4 * p);
      const f32x4 xq = row4<DK + 4>(sm.qP, rr, 16 * m + 4 * p);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        X = mfma_f32(xk[e], S_acc[m][e], X);
        O = mfma_f32(xq[e], S_acc[m][e], O);
      }
    }
    // this lane's values and betas, read before the barrier: the next block's step 1
    // rewrites them once every wavefront has passed it
    const int vc = 16 * wave + rr;
    f32x4 vv, bb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vv[e] = sm.v[4 * p + e][vc];
      bb[e] = sm.beta[4 * p + e];
    }
    __syncthreads();  // A_qk and Tm are in LDS
    // 5. V' = Tm Diag(beta) (V - X): the residual tile is the B operand over tokens 4 p + e
    f32x4 Rb;
#pragma unroll
    for (int e = 0; e < 4; ++e) Rb[e] = bb[e] * (vv[e] - X[e]);
    const f32x4 tmr = row4<kB + 4>(sm.tm, rr, 4 * p);
    const f32x4 aqr = row4<kB + 4>(sm.aqk, rr, 4 * p);
    f32x4 Vp = zero4();
#pragma unroll
    for (int e = 0; e < 4; ++e) Vp = mfma_f32(tmr[e], Rb[e], Vp);
    // O += A_qk V'
#pragma unroll
    for (int e = 0; e < 4; ++e) O = mfma_f32(aqr[e], Vp[e], O);
    if (a.o) {
      TIn* o = static_cast<TIn*>(a.o);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * p + e;
        if (t < nt) o[(row0 + kB * b + t) * DV + col] = from_f32<TIn>(O[e]);
      }
    }
    // S <- Diag(e^{G_15}) S + (K e^{G_15 - G})^T V'
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      f32x4 s_ = S_acc[m];
      const f32x4 tt = *reinterpret_cast<const f32x4*>(&sm.tot[16 * m + 4 * p]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s_[e] *= tt[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) s_ = mfma_f32(sm.kE[4 * p + e][16 * m + rr], Vp[e], s_);
      S_acc[m] = s_;
    }
    // the next block's step 1 overwrites only the raw inputs, which every wavefront has read
    // before the barrier of step 4; its steps 2 to 4 rewrite the rest after a barrier that
    // every wavefront passes only after this step
  }
  if (a.sT) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a.sT[mat + (size_t)(16 * m + 4 * p + e) * DV + col] = S_acc[m][e];
  }
}

template <int DK, typename TIn>
hipError_t launch_dk(const ChunkArgs& a, bool per_channel, hipStream_t stream) {
  const int groups = a.dv / kCols;
  const unsigned grid = (unsigned)((size_t)a.N * a.H * groups);
  if (grid == 0) return hipSuccess;
  const bool gdr2 = a.erase != nullptr;
  if (per_channel) {
    if (gdr2) chunk_f32mma_kernel<DK, TIn, true, true><<<grid, kThreads, 0, stream>>>(a, groups);
    else chunk_f32mma_kernel<DK, TIn, true, false><<<grid, kThreads, 0, stream>>>(a, groups);
  } else {
    if (gdr2) chunk_f32mma_kernel<DK, TIn, false, true><<<grid, kThreads, 0, stream>>>(a, groups);
    else chunk_f32mma_kernel<DK, TIn, false, false><<<grid, kThreads, 0, stream>>>(a, groups);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_f32(const ChunkArgs& a, bool bf16_io, bool per_channel,
                            hipStream_t stream) {
  if ((a.dk != 64 && a.dk != 128) || (a.dv != 64 && a.dv != 128)) return hipErrorInvalidValue;
  if (a.dk == 128)
    return bf16_io ? launch_dk<128, bf16>(a, per_channel, stream)
                   : launch_dk<128, float>(a, per_channel, stream);
  return bf16_io ? launch_dk<64, bf16>(a, per_channel, stream)
                 : launch_dk<64, float>(a, per_channel, stream);
}

}  // namespace kda
