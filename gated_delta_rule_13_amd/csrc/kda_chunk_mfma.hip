// Fused chunked forward on the CDNA4 matrix cores (bf16 operands, fp32 accumulate):
// the kda_chunk_fwd path for bf16 inputs with dk = 128.
//
// Method: the chunkwise form of "Token Mixer I", section "Kimi Delta Attention" (WY
// representation, UT transform, inter-chunk state update, chunk output), applied with a
// chunk of 16 tokens so that every bf16 operand stays within [e^-80, e^80] (the log-decay
// is at least -5 per token, so 16 tokens decay by at most e^-80). For a 16-token block
// starting after the state S (dk x dv), per key channel c and token t of the block:
//   P_t = exp(G_t - G_0) (decay from the block start through t, a prefix product of alpha),
//   E_t = exp(G_16 - G_t) (decay from after t to the block end), tot = exp(G_16 - G_0),
//   A_qk[i, j] = sum_c (q_i P_i)(k_j / P_j)   (j <= i)      A_kk likewise with k_i, j < i,
//   Tm = (I + Diag(beta) A_kk)^-1,   V' = Tm Diag(beta) (V - (K P) S)   (the pages' U - W S),
//   O  = (Q P) S + A_qk V',          S <- Diag(tot) S + (K E)^T V'.
// Every factor above is <= 1 except k / P (<= e^80 |k|), and every product of two of them
// is the exact exp(G_i - G_j) weighting, so no quantity is divided by a small decay.
//
// Layout: one workgroup per chain (sequence, head) with NW = dv / 16 wavefronts (8 for
// dv = 128, two per SIMD); wavefront w owns value columns [16 w, 16 w + 16) of the state
// for the whole sequence, held in matrix-core accumulator registers. The sequence is
// processed 64 tokens (four 16-token blocks) at a time: all wavefronts first compute the
// decay products and the bf16 operands of the four blocks into LDS; wavefronts 0..3 then
// compute the 16 x 16 A_qk / A_kk tile of one block each and invert its (I + A_kk) on the
// fp32 matrix cores; finally every wavefront runs the four blocks' state steps for its
// own columns. The next 64 tokens are loaded into registers during those state steps.
//
// Matrix-core operand layouts used (lane l, r = l % 16, p = l / 16):
//   16x16x32 bf16: A[r][8p + i], B[8p + i][r] (i < 8); D[4p + e][r] (e < 4)
//   16x16x16 bf16: A[r][4p + i], B[4p + i][r] (i < 4); D[4p + e][r]
//   16x16x4  fp32: A[r][p], B[p][r]; D[4p + e][r]
// The D layout of one product is the B layout of a 16x16x16 product, which chains the
// UT solve and the state update in registers. The contraction of the 16x16x32 products
// over channels is permuted (k = 8p + i <-> channel 32s + 16(i/4) + 4p + i%4) so that two
// D tiles of the state form one B operand without moving data between lanes.
#include <stddef.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

#ifndef KDA_NW128
#define KDA_NW128 8  // wavefronts per workgroup for dv = 128 (each owns 128 / (16 NW) tiles)
#endif

constexpr int kC = 64;         // tokens loaded and prepared at a time (four blocks)
constexpr int kDK = 128;       // key head size of this kernel
constexpr int kLDK = kDK + 8;  // padded LDS row (bf16) of [token][channel] tiles
constexpr int kLDT = kC + 8;   // padded LDS row (bf16) of [channel][token] tiles

struct Smem {
  bf16 qr[kC][kLDK];      // q * P
  bf16 kr[kC][kLDK];      // k * P
  bf16 kd[kC][kLDK];      // k / P
  bf16 kcT[kDK][kLDT];    // (k * E)^T
  bf16 vT[128][kLDT];     // V^T (value column, token)
  bf16 aqk[4][16][24];    // A_qk of each block (lower, diagonal included)
  bf16 tdiag[4][16][24];  // (I + Diag(beta) A_kk)^-1 of each block
  float tot[4][kDK];      // decay over each block
  float beta[kC];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget of one CU");
static_assert(offsetof(Smem, kcT) % 16 == 0 && offsetof(Smem, vT) % 16 == 0 &&
                  offsetof(Smem, aqk) % 16 == 0 && offsetof(Smem, tdiag) % 16 == 0 &&
                  offsetof(Smem, tot) % 16 == 0,
              "vector LDS accesses need 16-byte aligned arrays");
static_assert((kLDK * 2) % 16 == 0 && (kLDT * 2) % 16 == 0, "row pitch must keep alignment");

// LDS-only barrier: waits for this wavefront's LDS operations, not for its global loads
// (the prefetch of the next tokens stays in flight across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 pack4(f32x4 v) { return __builtin_convertvector(v, bf16x4); }
__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
  return pack4(f32x4{a, b, c, d});
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = a[i];
    r[4 + i] = b[i];
  }
  return r;
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// CPT consecutive bf16 values packed in registers (CPT = 2 or 4).
template <int CPT>
struct BfVec {
  typedef __attribute__((__vector_size__(CPT * sizeof(__bf16)))) __bf16 type;
};
template <int CPT>
struct F32Vec {
  typedef __attribute__((__vector_size__(CPT * sizeof(float)))) float type;
};
template <int CPT>
__device__ __forceinline__ typename BfVec<CPT>::type pack_bf(const float* v) {
  typename F32Vec<CPT>::type f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) f[j] = v[j];
  return __builtin_convertvector(f, typename BfVec<CPT>::type);
}
template <int CPT>
__device__ __forceinline__ void ld_f32(const float* src, float* dst) {
  if constexpr (CPT == 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = v[j];
  } else {
    const float2 v = *reinterpret_cast<const float2*>(src);
    dst[0] = v.x;
    dst[1] = v.y;
  }
}

// Work split of a workgroup with NW wavefronts. In the decay phase, wavefront w covers
// block I = w / (NW / 4) and channel segment w % (NW / 4); lane l covers the CPT channels
// CPT * (l % 32) + j of that segment and tokens 8 * (l / 32) + u of the block.
template <int NW, int NT = 1>
struct Split {
  static constexpr int kThreads = 64 * NW;
  static constexpr int CPT = 16 / NW;   // channels per thread in the decay phase
  static constexpr int SEGS = NW / 4;   // channel segments per block
  static constexpr int DV = 16 * NW * NT;
  __device__ static int block(int wave) { return wave / SEGS; }
  __device__ static int channel0(int wave, int lane) {
    return (wave % SEGS) * (kDK / SEGS) + CPT * (lane & 31);
  }
};

// Inputs of 64 tokens held in registers by one thread: q, k, g for 8 tokens x CPT
// channels (decay-phase split), two 8-column segments of v (token-major over the lanes,
// staged through LDS), and beta of one token (used by the first 64 threads).
template <int NW, int NT>
struct ChunkRegs {
  typename BfVec<Split<NW>::CPT>::type q[8];
  typename BfVec<Split<NW>::CPT>::type k[8];
  float g[8][Split<NW>::CPT];
  bf16x8 v[2 * NT];
  float beta;
};

// Loads tokens c0 .. c0 + nt - 1 (1 <= nt <= 64); positions past nt get the identity
// token (q = k = v = 0, g = 0, beta = 0).
template <int NW, int NT, bool PER_CHANNEL>
__device__ __forceinline__ void load_chunk(ChunkRegs<NW, NT>& r, const ChunkArgs& a,
                                           size_t row0, int c0, int nt, int tid) {
  using SP = Split<NW, NT>;
  constexpr int CPT = SP::CPT;
  typedef typename BfVec<CPT>::type bv;
  const int wave = tid >> 6, lane = tid & 63;
  const int I = SP::block(wave), ch0 = SP::channel0(wave, lane), hf = lane >> 5;
  const bf16* q = static_cast<const bf16*>(a.q);
  const bf16* k = static_cast<const bf16*>(a.k);
  const bf16* v = static_cast<const bf16*>(a.v);
  const bf16 zb = static_cast<bf16>(0.f);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int t = 16 * I + 8 * hf + u;
    const size_t row = row0 + c0 + t;
    if (t < nt) {
      r.q[u] = *reinterpret_cast<const bv*>(q + row * kDK + ch0);
      r.k[u] = *reinterpret_cast<const bv*>(k + row * kDK + ch0);
      if (PER_CHANNEL) {
        ld_f32<CPT>(a.g + row * kDK + ch0, r.g[u]);
      } else {
        const float gg = a.g[row];
#pragma unroll
        for (int j = 0; j < CPT; ++j) r.g[u][j] = gg;
      }
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        r.q[u][j] = zb;
        r.k[u][j] = zb;
        r.g[u][j] = 0.f;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int seg = tid + SP::kThreads * i;
    const int t = seg & 63, c8 = seg >> 6;
    if (t < nt) {
      r.v[i] = *reinterpret_cast<const bf16x8*>(v + (row0 + c0 + t) * SP::DV + 8 * c8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) r.v[i][j] = zb;
    }
  }
  const int tb = tid & 63;
  r.beta = tb < nt ? a.beta[row0 + c0 + tb] : 0.f;
}

// The bf16 operands of one thread's share of the 64 tokens, ready to be written to LDS:
// q P, k P, k / P per token (CPT channels), k E per channel (8 tokens), the decay over
// the block, and the staged v and beta.
template <int NW, int NT>
struct Prepped {
  typename BfVec<Split<NW>::CPT>::type qr[8], kr[8], kd[8];
  bf16x8 kc[Split<NW>::CPT];
  float tot[Split<NW>::CPT];
  bf16x8 v[2 * NT];
  float beta;
};

// Decay products inside the thread's block (tokens 8 hf + u, channels ch0 + j):
// P = exp(G_t - G_0) (prefix), E = exp(G_16 - G_t) (suffix after t), tot = P * E.
template <int NW, int NT>
__device__ __forceinline__ void prep(Prepped<NW, NT>& o, const ChunkRegs<NW, NT>& c, int hf) {
  constexpr int CPT = Split<NW>::CPT;
  float P[8][CPT], E[8][CPT], al[8][CPT], run[CPT], rs[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) run[j] = rs[j] = 1.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      al[u][j] = __expf(c.g[u][j]);
      run[j] *= al[u][j];
      P[u][j] = run[j];
    }
  }
#pragma unroll
  for (int u = 7; u >= 0; --u) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      E[u][j] = rs[j];
      rs[j] *= al[u][j];
    }
  }
  float other[CPT], rtot[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    other[j] = __shfl_xor(run[j], 32, 64);  // the other half block's product
    o.tot[j] = run[j] * other[j];
    rtot[j] = __builtin_amdgcn_rcpf(o.tot[j]);
  }
  float kcv[8][CPT];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float qr[CPT], kr[CPT], kd[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      // upper half: prefix times the lower half's product; lower half: suffix times
      // the upper half's product
      const float pp = hf ? P[u][j] * other[j] : P[u][j];
      const float ee = hf ? E[u][j] : E[u][j] * other[j];
      const float qv = static_cast<float>(c.q[u][j]);
      const float kv = static_cast<float>(c.k[u][j]);
      qr[j] = qv * pp;
      kr[j] = kv * pp;
      kcv[u][j] = kv * ee;
      kd[j] = kcv[u][j] * rtot[j];
    }
    o.qr[u] = pack_bf<CPT>(qr);
    o.kr[u] = pack_bf<CPT>(kr);
    o.kd[u] = pack_bf<CPT>(kd);
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const f32x4 lo = {kcv[0][j], kcv[1][j], kcv[2][j], kcv[3][j]};
    const f32x4 hi = {kcv[4][j], kcv[5][j], kcv[6][j], kcv[7][j]};
    o.kc[j] = cat8(pack4(lo), pack4(hi));
  }
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) o.v[i] = c.v[i];
  o.beta = c.beta;
}

template <int NW, int NT>
__device__ __forceinline__ void write_prepped(Smem& sm, const Prepped<NW, NT>& o, int tid) {
  using SP = Split<NW, NT>;
  constexpr int CPT = SP::CPT;
  typedef typename BfVec<CPT>::type bv;
  const int wave = tid >> 6, lane = tid & 63;
  const int I = SP::block(wave), ch0 = SP::channel0(wave, lane), hf = lane >> 5;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int t = 16 * I + 8 * hf + u;
    *reinterpret_cast<bv*>(&sm.qr[t][ch0]) = o.qr[u];
    *reinterpret_cast<bv*>(&sm.kr[t][ch0]) = o.kr[u];
    *reinterpret_cast<bv*>(&sm.kd[t][ch0]) = o.kd[u];
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    *reinterpret_cast<bf16x8*>(&sm.kcT[ch0 + j][16 * I + 8 * hf]) = o.kc[j];
    if (hf == 0) sm.tot[I][ch0 + j] = o.tot[j];
  }
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int seg = tid + SP::kThreads * i;
    const int t = seg & 63, c8 = seg >> 6;
#pragma unroll
    for (int j = 0; j < 8; ++j) sm.vT[8 * c8 + j][t] = o.v[i][j];
  }
  if (tid < kC) sm.beta[tid] = o.beta;
}

// 16 x 16 fp32 products on the matrix cores with X in row layout (lane 16p + r holds
// X[r][4p + e]) and Y in column layout (holds Y[4p + e][r], the accumulator layout); the
// contraction index of step s is 4p + s, which both layouts hold as element s.
// mm_col returns X Y in column layout; mm_row returns X Y in row layout, computed as the
// column layout of Y^T X^T.
__device__ __forceinline__ f32x4 mm_col(const f32x4& xr, const f32x4& yc) {
  f32x4 acc = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_f32(xr[s], yc[s], acc);
  return acc;
}
__device__ __forceinline__ f32x4 mm_row(const f32x4& xr, const f32x4& yc) {
  f32x4 acc = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_f32(yc[s], xr[s], acc);
  return acc;
}

// The A_qk / A_kk tile of block I and the inverse of its (I + N), N = Diag(beta) A_kk
// strictly lower. N is nilpotent (N^16 = 0), so (I + N)^-1 = (I - N)(I + N^2)(I + N^4)
// (I + N^8) exactly; the factors are polynomials in N and commute, which lets every
// product take its left factor in row layout and its right factor in column layout.
__device__ __forceinline__ void block_tiles(Smem& sm, int I, int rr, int p) {
  bf16x8 bq[4], bk[4], bc[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = 32 * ks + 8 * p;
    bq[ks] = *reinterpret_cast<const bf16x8*>(&sm.qr[16 * I + rr][ch]);
    bk[ks] = *reinterpret_cast<const bf16x8*>(&sm.kr[16 * I + rr][ch]);
    bc[ks] = *reinterpret_cast<const bf16x8*>(&sm.kd[16 * I + rr][ch]);
  }
  f32x4 accq = zero4(), acck = zero4(), acct = zero4();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    accq = mfma32(bq[ks], bc[ks], accq);   // A_qk[i][j], lane holds i = 4p + e, j = rr
    acck = mfma32(bk[ks], bc[ks], acck);   // A_kk[i][j]
    acct = mfma32(bc[ks], bk[ks], acct);   // A_kk[j][i]: lane holds A_kk[rr][4p + e]
  }
  f32x4 nc, nr;
  const float brr = sm.beta[16 * I + rr];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * p + e;
    sm.aqk[I][i][rr] = static_cast<bf16>(rr <= i ? accq[e] : 0.f);
    nc[e] = rr < i ? sm.beta[16 * I + i] * acck[e] : 0.f;   // N[i][rr]
    nr[e] = i < rr ? brr * acct[e] : 0.f;                    // N[rr][i]
  }
  const f32x4 n2c = mm_col(nr, nc), n2r = mm_row(nr, nc);
  const f32x4 n4c = mm_col(n2r, n2c), n4r = mm_row(n2r, n2c);
  const f32x4 n8r = mm_row(n4r, n4c);
  const f32x4 nn2c = mm_col(nr, n2c);
  f32x4 y1;
#pragma unroll
  for (int e = 0; e < 4; ++e) y1[e] = (4 * p + e == rr ? 1.f : 0.f) - nc[e] + n2c[e] - nn2c[e];
  const f32x4 t1 = mm_col(n4r, y1);
  f32x4 y2;
#pragma unroll
  for (int e = 0; e < 4; ++e) y2[e] = y1[e] + t1[e];
  const f32x4 t2 = mm_col(n8r, y2);
#pragma unroll
  for (int e = 0; e < 4; ++e) sm.tdiag[I][4 * p + e][rr] = static_cast<bf16>(y2[e] + t2[e]);
}

template <int NW, int NT, bool PER_CHANNEL>
__global__ __launch_bounds__(64 * NW) void chunk_mfma_kernel(ChunkArgs a) {
  using SP = Split<NW, NT>;
  constexpr int DV = SP::DV;
  __shared__ __align__(16) Smem sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hf = lane >> 5;                 // decay phase: token half of the block
  const int rr = lane & 15, p = lane >> 4;  // matrix-core phases

  const int chain = blockIdx.x;
  const int n = chain / a.H;
  const int h = chain % a.H;
  const TokenRange tr = token_range(a.cu, n, a.T);
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0;
  const size_t state_off = ((size_t)n * a.H + h) * kDK * DV;

  // state S[channel][column] of this wavefront's NT column tiles, accumulator layout:
  // S_acc[j][m][e] = S[16 m + 4 p + e][16 (NT wave + j) + rr]
  f32x4 S_acc[NT][8];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int col = 16 * (NT * wave + j) + rr;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S_acc[j][m][e] =
            a.s0 ? a.s0[state_off + (size_t)(16 * m + 4 * p + e) * DV + col] : 0.f;
  }

  ChunkRegs<NW, NT> cur;
  if (tr.len > 0) load_chunk<NW, NT, PER_CHANNEL>(cur, a, row0, 0, min(kC, tr.len), tid);

  for (int c0 = 0; c0 < tr.len; c0 += kC) {
    const int nt = min(kC, tr.len - c0);
    lds_barrier();  // the previous tokens' state steps are done with LDS
    {
      Prepped<NW, NT> pre;
      prep<NW, NT>(pre, cur, hf);
      write_prepped<NW, NT>(sm, pre, tid);
    }
    lds_barrier();

    // ---- per block: A_qk and A_kk tiles, and the inverse of (I + Diag(beta) A_kk)
    if (wave < 4) block_tiles(sm, wave, rr, p);
    lds_barrier();

    // every input of these tokens is in LDS now: fetch the next ones while computing
    const bool has_next = c0 + kC < tr.len;
    if (has_next)
      load_chunk<NW, NT, PER_CHANNEL>(cur, a, row0, c0 + kC, min(kC, tr.len - c0 - kC), tid);

    // ---- the four blocks' state steps for this wavefront's column tiles
    bf16* o = static_cast<bf16*>(a.o);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      // B operands of S (bf16), contraction permuted over channels
      bf16x8 sb[NT][4];
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          sb[j][ks] = cat8(pack4(S_acc[j][2 * ks]), pack4(S_acc[j][2 * ks + 1]));
      // X = (K P) S and O = (Q P) S
      f32x4 X[NT], Oc[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) X[j] = Oc[j] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16* kr_ = &sm.kr[16 * I + rr][32 * ks + 4 * p];
        const bf16* qr_ = &sm.qr[16 * I + rr][32 * ks + 4 * p];
        const bf16x8 ak = cat8(*reinterpret_cast<const bf16x4*>(kr_),
                               *reinterpret_cast<const bf16x4*>(kr_ + 16));
        const bf16x8 aq = cat8(*reinterpret_cast<const bf16x4*>(qr_),
                               *reinterpret_cast<const bf16x4*>(qr_ + 16));
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          X[j] = mfma32(ak, sb[j][ks], X[j]);
          Oc[j] = mfma32(aq, sb[j][ks], Oc[j]);
        }
      }
      // V' = Tm Diag(beta) (V - X)
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * I + 4 * p]);
      const bf16x4 tI = *reinterpret_cast<const bf16x4*>(&sm.tdiag[I][rr][4 * p]);
      const bf16x4 aI = *reinterpret_cast<const bf16x4*>(&sm.aqk[I][rr][4 * p]);
      bf16x4 vp[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int col = 16 * (NT * wave + j) + rr;
        const bf16x4 vv = *reinterpret_cast<const bf16x4*>(&sm.vT[col][16 * I + 4 * p]);
        f32x4 R;
#pragma unroll
        for (int e = 0; e < 4; ++e) R[e] = bt[e] * (static_cast<float>(vv[e]) - X[j][e]);
        vp[j] = pack4(mfma16(tI, pack4(R), zero4()));
        // O += A_qk V'
        const bf16x4 ob = pack4(mfma16(aI, vp[j], Oc[j]));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + 4 * p + e;
          if (t < nt) o[(row0 + c0 + t) * DV + col] = ob[e];
        }
      }
      // S <- Diag(tot) S + (K E)^T V'
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const f32x4 dc = *reinterpret_cast<const f32x4*>(&sm.tot[I][16 * m + 4 * p]);
        const bf16x4 ac = *reinterpret_cast<const bf16x4*>(&sm.kcT[16 * m + rr][16 * I + 4 * p]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          f32x4 s_ = S_acc[j][m];
#pragma unroll
          for (int e = 0; e < 4; ++e) s_[e] *= dc[e];
          S_acc[j][m] = mfma16(ac, vp[j], s_);
        }
      }
    }
  }

  if (a.sT) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int col = 16 * (NT * wave + j) + rr;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.sT[state_off + (size_t)(16 * m + 4 * p + e) * DV + col] = S_acc[j][m][e];
    }
  }
}

template <int NW, int NT, bool PER_CHANNEL>
hipError_t launch_nw(const ChunkArgs& a, hipStream_t stream) {
  chunk_mfma_kernel<NW, NT, PER_CHANNEL><<<dim3(a.N * a.H), dim3(64 * NW), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supports(int dk, int dv) { return dk == kDK && (dv == 64 || dv == 128); }

hipError_t launch_chunk_mfma(const ChunkArgs& a, bool per_channel, hipStream_t stream) {
  if (!chunk_mfma_supports(a.dk, a.dv)) return hipErrorInvalidValue;
  if (a.dv == 128)
    return per_channel ? launch_nw<KDA_NW128, 8 / KDA_NW128, true>(a, stream)
                       : launch_nw<KDA_NW128, 8 / KDA_NW128, false>(a, stream);
  return per_channel ? launch_nw<4, 1, true>(a, stream) : launch_nw<4, 1, false>(a, stream);
}

}  // namespace kda
