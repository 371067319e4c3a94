// Chunked forward on the fp32 matrix cores (16x16x4 fp32 products): the kda_chunk_fwd path
// for float32 inputs, for dk = 64, and for whatever the bf16 kernel does not take (dv = 64
// chains past 2^22 tokens, long axes without a workspace). Every operand and every product is
// fp32; bf16 inputs are widened on load and the outputs rounded on store.
//
// The algorithm is the chunkwise form of "Token Mixer I", section "Kimi Delta Attention"
// (WY representation, UT transform, inter-chunk state update, chunk output), taken over
// blocks of 16 tokens. With G_t the block-local inclusive cumulative log decay per key
// channel and G_15 its value at the block's end:
//   A_qk[i][j] = sum_c q_i[c] k_j[c] e^{G_i[c] - G_j[c]}           (j <= i)
//   A_kk[i][j] = sum_c k_i[c] k_j[c] e^{G_i[c] - G_j[c]}           (j <  i)
//   Tm = (I + Diag(beta) A_kk)^-1,   V' = Tm Diag(beta) (V - (K e^G) S)
//   O  = (Q e^G) S + A_qk V',        S <- Diag(e^{G_15}) S + (K e^{G_15 - G})^T V'
// The decay weight of A_qk and A_kk is split at the block's end,
// e^{G_i - G_j} = (e^{G_i} / e^{G_15}) e^{G_15 - G_j}: with g >= -5 the left factor lies in
// [1, e^75] and every other factor in [e^-80, 1], all inside the fp32 range, so nothing is
// divided by a decay smaller than e^-80. Tm is the exact nilpotent product
// (I - N)(I + N^2)(I + N^4)(I + N^8) on the matrix cores.
//
// Gated Delta Rule-2 ("Token Mixer I", section "Gated DeltaNet-2"): the read side takes the
// erase-gated keys b * k in A_kk and in the prediction, beta is 1, and the values are the
// write-gated w * V.
//
// One workgroup per (chain, 64 value columns), six wavefronts in two roles:
//  - two prep wavefronts, one per 16-token block of the next 32 tokens: each loads its block,
//    forms the cumulative decay and the decayed operands in LDS, then A_qk and the inverse;
//  - four state wavefronts, each owning 16 value columns and their dk x 16 slice of S in
//    accumulator registers, run the two blocks of the current 32 tokens from those operands.
// The operands of 32 tokens are double-buffered; one workgroup barrier per 32 tokens. Plain
// 64-bit addressing: any T.
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

constexpr int kB = 16;            // tokens per block
constexpr int kNB = 2;            // blocks per step (one per prep wavefront)
constexpr int kStateWaves = 4;
constexpr int kThreads = 64 * (kStateWaves + kNB);
constexpr int kCols = 16 * kStateWaves;  // value columns per workgroup

// Operands of one step (kNB blocks), written by the prep wavefronts.
template <int DK>
struct F32Stage {
  float qP[kNB][kB][DK + 4];      // q e^G
  float kP[kB * kNB][DK + 4];     // (b *) k e^G, block-major rows
  float kE[kNB][kB][DK + 1];      // k e^{G_15 - G}
  float tot[kNB][DK];             // e^{G_15}
  float aqk[kNB][kB][kB + 4];     // A_qk (lower, diagonal included)
  float tm[kNB][kB][kB + 4];      // Tm
  float v[kNB][kB][kCols + 1];    // V, or w * V, of the workgroup's columns
  float beta[kNB][kB];
};
template <int DK>
struct F32Smem {
  F32Stage<DK> st[2];
  float nn[kNB][kB][kB + 1];      // Diag(beta) A_kk of each prep wavefront, for its transpose
};
static_assert(sizeof(F32Smem<128>) <= 160 * 1024, "LDS budget of one CU");
static_assert(offsetof(F32Stage<128>, kP) % 16 == 0 && offsetof(F32Stage<128>, kE) % 16 == 0 &&
                  offsetof(F32Stage<128>, tot) % 16 == 0 &&
                  offsetof(F32Stage<128>, aqk) % 16 == 0 &&
                  offsetof(F32Stage<128>, tm) % 16 == 0 && sizeof(F32Stage<128>) % 16 == 0 &&
                  offsetof(F32Stage<64>, kP) % 16 == 0 && offsetof(F32Stage<64>, kE) % 16 == 0 &&
                  offsetof(F32Stage<64>, tot) % 16 == 0 &&
                  offsetof(F32Stage<64>, aqk) % 16 == 0 &&
                  offsetof(F32Stage<64>, tm) % 16 == 0 && sizeof(F32Stage<64>) % 16 == 0,
              "16-byte LDS reads need aligned rows");

// A prep lane holds four consecutive channels (4 cq .. 4 cq + 3) of kTPL consecutive tokens
// (kTPL tg .. ), so that a token row's channels lie in consecutive lanes.
template <int DK>
struct PrepLayout {
  static constexpr int kCL = DK / 4;      // lanes per token group
  static constexpr int kTG = 64 / kCL;    // token groups
  static constexpr int kTPL = kB / kTG;   // tokens per lane
};

// One prep wavefront's block inputs in registers.
template <int DK, bool GDR2>
struct PrepRegs {
  static constexpr int N = PrepLayout<DK>::kTPL;
  f32x4 q[N], k[N], g[N], e[GDR2 ? N : 1];
  f32x4 v[4], w[GDR2 ? 4 : 1];           // token lane / 4, columns 16 (lane % 4) ..
  float beta;                            // token lane (lanes below 16)
};

template <typename TIn>
__device__ __forceinline__ f32x4 ld4(const TIn* p) {
  if constexpr (sizeof(TIn) == 4) {
    return *reinterpret_cast<const f32x4*>(p);
  } else {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
                 static_cast<float>(x[3])};
  }
}

// Loads the block of nt valid tokens starting at row `row` (tokens past nt read as identity
// tokens: zero q, k, v, g and beta).
template <int DK, typename TIn, bool PER_CHANNEL, bool GDR2>
__device__ __forceinline__ void prep_load(PrepRegs<DK, GDR2>& r, const ChunkArgs& a,
                                          size_t row, int nt, int col0, int lane) {
  using L = PrepLayout<DK>;
  const int cq = lane % L::kCL, tg = lane / L::kCL;
  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
  const TIn* v = static_cast<const TIn*>(a.v);
#pragma unroll
  for (int u = 0; u < L::kTPL; ++u) {
    const int t = L::kTPL * tg + u;
    const bool ok = t < nt;
    const size_t off = (row + t) * DK + 4 * cq;
    r.q[u] = ok ? ld4<TIn>(q + off) : zero4();
    r.k[u] = ok ? ld4<TIn>(k + off) : zero4();
    if constexpr (PER_CHANNEL) {
      r.g[u] = ok ? *reinterpret_cast<const f32x4*>(a.g + off) : zero4();
    } else {
      const float gv = ok ? a.g[row + t] : 0.f;
      r.g[u] = f32x4{gv, gv, gv, gv};
    }
    if constexpr (GDR2) r.e[u] = ok ? *reinterpret_cast<const f32x4*>(a.erase + off) : zero4();
  }
  const int tv = lane / 4, cv = 16 * (lane % 4);
  const bool okv = tv < nt;
  const size_t offv = (row + tv) * a.dv + col0 + cv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[i] = okv ? ld4<TIn>(v + offv + 4 * i) : zero4();
    if constexpr (GDR2)
      r.w[i] = okv ? *reinterpret_cast<const f32x4*>(a.write + offv + 4 * i) : zero4();
  }
  r.beta = (!GDR2 && lane < nt) ? a.beta[row + lane] : 0.f;
}

// The cumulative decay and the decayed operands of block j of a stage (from registers).
template <int DK, bool GDR2>
__device__ __forceinline__ void prep_operands(F32Stage<DK>& st, const PrepRegs<DK, GDR2>& r,
                                              int j, int lane) {
  using L = PrepLayout<DK>;
  const int cq = lane % L::kCL, tg = lane / L::kCL;
  // cumulative log decay: within the lane's tokens, then the lower token groups' totals
  f32x4 G[L::kTPL];
  G[0] = r.g[0];
#pragma unroll
  for (int u = 1; u < L::kTPL; ++u) G[u] = G[u - 1] + r.g[u];
  const f32x4 mine = G[L::kTPL - 1];
  f32x4 before = zero4(), all = zero4();
#pragma unroll
  for (int gi = 0; gi < L::kTG; ++gi) {
    f32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = __shfl(mine[c], cq + L::kCL * gi, 64);
    if (gi < tg) before += o;
    all += o;
  }
  // e^{G_15} of the lane's channels
  f32x4 tot;
#pragma unroll
  for (int c = 0; c < 4; ++c) tot[c] = __expf(all[c]);
  if (tg == 0) *reinterpret_cast<f32x4*>(&st.tot[j][4 * cq]) = tot;
#pragma unroll
  for (int u = 0; u < L::kTPL; ++u) {
    const int t = L::kTPL * tg + u;
    f32x4 qp, kp, ke;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float Gt = G[u][c] + before[c];
      const float eG = __expf(Gt);
      const float kr = GDR2 ? r.e[u][c] * r.k[u][c] : r.k[u][c];  // the read-side key
      qp[c] = r.q[u][c] * eG;
      kp[c] = kr * eG;
      ke[c] = r.k[u][c] * __expf(all[c] - Gt);
    }
    *reinterpret_cast<f32x4*>(&st.qP[j][t][4 * cq]) = qp;
    *reinterpret_cast<f32x4*>(&st.kP[kB * j + t][4 * cq]) = kp;
#pragma unroll
    for (int c = 0; c < 4; ++c) st.kE[j][t][4 * cq + c] = ke[c];
  }
  const int tv = lane / 4, cv = 16 * (lane % 4);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      st.v[j][tv][cv + 4 * i + c] = GDR2 ? r.w[i][c] * r.v[i][c] : r.v[i][c];
  if (lane < kB) st.beta[j][lane] = GDR2 ? 1.f : r.beta;
}

// A_qk and Tm of block j (the operands of the block are in LDS, written by this wavefront).
// A_qk = (Q e^G / e^{G_15}) (K e^{G_15 - G})^T and A_kk likewise with the read-side key.
template <int DK>
__device__ __forceinline__ void prep_tiles(F32Stage<DK>& st, float (*nn)[kB + 1], int j,
                                           int rr, int p) {
  constexpr int NM = DK / 16;
  f32x4 aq = zero4(), ak = zero4();
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int c0 = 16 * m + 4 * p;
    const f32x4 ttc = *reinterpret_cast<const f32x4*>(&st.tot[j][c0]);
    const f32x4 xq = *reinterpret_cast<const f32x4*>(&st.qP[j][rr][c0]);
    const f32x4 xk = *reinterpret_cast<const f32x4*>(&st.kP[kB * j + rr][c0]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float rt = __builtin_amdgcn_rcpf(ttc[e]);
      const float y = st.kE[j][rr][c0 + e];
      aq = mfma_f32(xq[e] * rt, y, aq);
      ak = mfma_f32(xk[e] * rt, y, ak);
    }
  }
  // aq[e] = A_qk[4 p + e][rr], ak[e] = A_kk[4 p + e][rr]
  f32x4 nc, nr;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * p + e;
    st.aqk[j][i][rr] = rr <= i ? aq[e] : 0.f;
    nc[e] = rr < i ? st.beta[j][i] * ak[e] : 0.f;  // N[i][rr]
    nn[i][rr] = nc[e];
  }
  wave_lds_fence();
#pragma unroll
  for (int e = 0; e < 4; ++e) nr[e] = nn[rr][4 * p + e];  // N[rr][4 p + e]
  const f32x4 inv = unit_lower_inverse(nc, nr, rr, p);
#pragma unroll
  for (int e = 0; e < 4; ++e) st.tm[j][4 * p + e][rr] = inv[e];
}

template <int LD>
__device__ __forceinline__ f32x4 row4(const float (*x)[LD], int r, int c) {
  return *reinterpret_cast<const f32x4*>(&x[r][c]);
}

template <int DK, typename TIn, bool PER_CHANNEL, bool GDR2>
__global__ __launch_bounds__(kThreads) void chunk_f32mma_kernel(ChunkArgs a, int groups) {
  constexpr int NM = DK / 16;       // row tiles of S
  __shared__ __align__(16) F32Smem<DK> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rr = lane & 15, p = lane >> 4;
  const int chain = blockIdx.x / groups, grp = blockIdx.x % groups;
  const int n = chain / a.H, h = chain % a.H;
  const int DV = a.dv;
  const int col0 = grp * kCols;           // the workgroup's first value column
  const TokenRange tr = token_range(a.cu, n, a.T);
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0;
  const int nblk = (tr.len + kB - 1) / kB;
  const int nsteps = (nblk + kNB - 1) / kNB;

  if (wave >= kStateWaves) {
    // prep wavefront j: block kNB s + j of every step s, one step ahead of the state
    const int j = wave - kStateWaves;
    PrepRegs<DK, GDR2> r;
    auto load = [&](int s) {
      const int t0 = kB * (kNB * s + j);
      prep_load<DK, TIn, PER_CHANNEL, GDR2>(r, a, row0 + t0, tr.len - t0, col0, lane);
    };
    if (nsteps > 0) {
      load(0);
      prep_operands<DK, GDR2>(sm.st[0], r, j, lane);
      if (nsteps > 1) load(1);
      wave_lds_fence();
      prep_tiles<DK>(sm.st[0], sm.nn[j], j, rr, p);
    }
    lds_barrier();
    for (int s = 0; s < nsteps; ++s) {
      if (s + 1 < nsteps) {
        F32Stage<DK>& st = sm.st[(s + 1) & 1];
        prep_operands<DK, GDR2>(st, r, j, lane);
        if (s + 2 < nsteps) load(s + 2);  // in flight during the tiles and the barrier
        wave_lds_fence();
        prep_tiles<DK>(st, sm.nn[j], j, rr, p);
      }
      lds_barrier();
    }
    return;
  }

  // state wavefront: value columns col .. of the workgroup's
  const int col = col0 + 16 * wave + rr;
  const int vc = 16 * wave + rr;
  const size_t mat = ((size_t)n * a.H + h) * DK * DV;
  // S_acc[m][e] = S[16 m + 4 p + e][col]
  f32x4 S_acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S_acc[m][e] = a.s0 ? a.s0[mat + (size_t)(16 * m + 4 * p + e) * DV + col] : 0.f;
  lds_barrier();  // the first step's operands are in LDS
  TIn* o = static_cast<TIn*>(a.o);
  for (int s = 0; s < nsteps; ++s) {
    const F32Stage<DK>& st = sm.st[s & 1];
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      const int t0 = kB * (kNB * s + j);  // the block's first token
      // X = ((b *) K e^G) S and (Q e^G) S
      f32x4 X = zero4(), O = zero4();
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const f32x4 xk = row4<DK + 4>(st.kP, kB * j + rr, 16 * m + 4 * p);
        const f32x4 xq = row4<DK + 4>(st.qP[j], rr, 16 * m + 4 * p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          X = mfma_f32(xk[e], S_acc[m][e], X);
          O = mfma_f32(xq[e], S_acc[m][e], O);
        }
      }
      // V' = Tm Diag(beta) (V - X): the residual tile is the B operand over tokens 4 p + e
      f32x4 Rb;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Rb[e] = st.beta[j][4 * p + e] * (st.v[j][4 * p + e][vc] - X[e]);
      const f32x4 tmr = row4<kB + 4>(st.tm[j], rr, 4 * p);
      const f32x4 aqr = row4<kB + 4>(st.aqk[j], rr, 4 * p);
      f32x4 Vp = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) Vp = mfma_f32(tmr[e], Rb[e], Vp);
      // O += A_qk V'
#pragma unroll
      for (int e = 0; e < 4; ++e) O = mfma_f32(aqr[e], Vp[e], O);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 4 * p + e;
        if (t < tr.len) o[(row0 + t) * DV + col] = from_f32<TIn>(O[e]);
      }
      // S <- Diag(e^{G_15}) S + (K e^{G_15 - G})^T V'
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        f32x4 s_ = S_acc[m];
        const f32x4 tt = *reinterpret_cast<const f32x4*>(&st.tot[j][16 * m + 4 * p]);
#pragma unroll
        for (int e = 0; e < 4; ++e) s_[e] *= tt[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) s_ = mfma_f32(st.kE[j][4 * p + e][16 * m + rr], Vp[e], s_);
        S_acc[m] = s_;
      }
    }
    lds_barrier();  // this stage is read; the next one is written
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
