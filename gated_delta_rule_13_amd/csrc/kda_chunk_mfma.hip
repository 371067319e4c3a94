// Fused chunked forward on the CDNA4 matrix cores (bf16 operands, fp32 accumulate):
// the kda_chunk_fwd path for bf16 inputs with dk = 128.
//
// Method: the chunkwise form of "Token Mixer I", section "Kimi Delta Attention"
// (WY representation, UT transform, inter-chunk state update, chunk output), with the
// chunk of C = 64 tokens cut into four 16-token sub-blocks so that every bf16 operand
// stays within [e^-80, e^80] (the log-decay is at least -5 per token):
//
//   Notation per chunk, per key channel c: alpha_t = exp(g_t); for sub-block I,
//   R_I = G just before the block (R_0 = 0), P_t = exp(G_t - R_I) (prefix product of
//   alpha inside the block), E_t = exp(R_{I+1} - G_t) (product of alpha after t inside the
//   block), tot_I = exp(R_{I+1} - R_I).
//   A_qk[i,j] = sum_c q_i k_j exp(G_i - G_j) (j <= i), A_kk likewise with k_i and a beta_i
//   row scale (j < i). Tile (I, J) of these C x C matrices is one matrix-core product:
//     row operand  (q or k) * P              (<= 1)
//     column operand, by tile:  J = I     : k / P                       (<= e^80)
//                               J = I - 1 : k * E                       (<= 1)
//                               J < I - 1 : k * E * prod_{J<I'<I} tot_I' (<= 1)
//   so that row * column = q_i k_j exp(G_i - G_j) exactly (up to rounding).
//   UT transform: Tm = (I + A_kk)^-1, never formed whole: the 16 x 16 diagonal blocks are
//   inverted by forward substitution in fp32, and V' = Tm Diag(beta) (V - K^ S) (the pages'
//   U - W S) is solved block by block:
//     V'_I = T_II (B_I - sum_{J<I} A_kk[I,J] V'_J),   B = Diag(beta)(V - K^ S).
//   Output and state:  O = Q^ S + A_qk V',   S <- Diag(exp G_C) S + K_dec^T V',
//   with Q^ = q exp(G), K^ = k exp(G), K_dec = k exp(G_C - G) (all <= 1).
//
// Layout: one workgroup of 4 wavefronts per chain (sequence, head); wavefront w owns
// value columns [w*16*NT, (w+1)*16*NT) of the state for the whole sequence. S lives in
// matrix-core accumulator registers between chunks; the intermediates of a chunk live
// in LDS only. Per chunk: the four 16-token sub-blocks are spread over the four
// wavefronts for the decay products, the ten (I, J) tiles of A_qk / A_kk are spread
// over the wavefronts, each wavefront inverts one diagonal block, and then every
// wavefront runs the state pass for its own columns. The next chunk's inputs are
// loaded into registers while the current chunk is processed.
//
// Matrix-core operand layouts used (lane l, r = l % 16, p = l / 16):
//   16x16x32 bf16: A[r][8p + i], B[8p + i][r] (i < 8); D[4p + e][r] (e < 4)
//   16x16x16 bf16: A[r][4p + i], B[4p + i][r] (i < 4); D[4p + e][r]
// The D layout of one product is the B layout of a 16x16x16 product, which is what
// chains the block substitution in registers. The contraction index of the 16x16x32
// products over channels / tokens is permuted (k = 8p + i <-> 32s + 16(i/4) + 4p + i%4)
// so that two D tiles form one B operand without moving data between lanes.
#include <stddef.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kC = 64;         // chunk length
constexpr int kDK = 128;       // key head size of this kernel
constexpr int kThreads = 256;  // four wavefronts
constexpr int kLDK = kDK + 8;  // padded LDS row (bf16) of [token][channel] tiles
constexpr int kLDT = kC + 8;   // padded LDS row (bf16) of [channel][token] and [token][token]

struct Smem {
  union {
    struct {                       // operands of the A_qk / A_kk tiles
      bf16 qr[kC][kLDK];           // q * P
      bf16 kr[kC][kLDK];           // k * P
      bf16 kc[48][kLDK];           // k * E, sub-blocks 0..2
      bf16 kd[kC][kLDK];           // k / P
      bf16 kfar[48][kLDK];         // k*E*tot_1 (blk 0), k*E*tot_2 (blk 1), k*E*tot_1*tot_2 (blk 0)
    } a;
    struct {                       // operands of the state pass
      bf16 qh[kC][kLDK];           // q exp(G)
      bf16 kh[kC][kLDK];           // k exp(G)
      bf16 kdecT[kDK][kLDT];       // (k exp(G_C - G))^T
      bf16 vT[128][kLDT];          // V^T (value column, token)
    } s;
  } x;
  bf16 akk_neg[kC][kLDT];          // -beta_i A_kk[i, j], j < i
  bf16 aqk[kC][kLDT];              // A_qk[i, j], j <= i
  bf16 tdiag[4][16][24];           // (I + A_kk[I, I])^-1
  float adiag[4][16][17];          // beta_i A_kk[i, j] inside the diagonal blocks (fp32)
  float tot[4][kDK];
  float egc[kDK];
  float beta[kC];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget of one CU");
static_assert(offsetof(Smem, akk_neg) % 16 == 0 && offsetof(Smem, aqk) % 16 == 0 &&
                  offsetof(Smem, tdiag) % 16 == 0 && offsetof(Smem, tot) % 16 == 0 &&
                  offsetof(Smem, egc) % 16 == 0,
              "vector LDS accesses need 16-byte aligned arrays");
static_assert((kLDK * 2) % 16 == 0 && (kLDT * 2) % 16 == 0, "row pitch must keep alignment");

// LDS-only barrier: waits for this wavefront's LDS operations, not for its global loads
// (the prefetch of the next chunk stays in flight across it).
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

__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = static_cast<bf16>(a);
  r[1] = static_cast<bf16>(b);
  r[2] = static_cast<bf16>(c);
  r[3] = static_cast<bf16>(d);
  return r;
}
__device__ __forceinline__ bf16x4 pack4(f32x4 v) { return pack4(v[0], v[1], v[2], v[3]); }

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

__device__ __forceinline__ void st4(bf16* p, f32x4 v) {
  *reinterpret_cast<bf16x4*>(p) = pack4(v);
}

// Inputs of one chunk held in registers by one thread. q, k, g: 8 tokens x 4 channels
// (sub-block = wavefront, half = lane / 32, channels 4 * (lane % 32) ...); v: 2 * NT
// segments of 8 consecutive value columns of one token, staged through LDS; beta: one
// token for the first 64 threads.
template <int NT>
struct ChunkRegs {
  bf16x4 q[8];
  bf16x4 k[8];
  f32x4 g[8];
  bf16x8 v[2 * NT];
  float beta;
};

template <int NT, bool PER_CHANNEL>
__device__ __forceinline__ void load_chunk(ChunkRegs<NT>& r, const ChunkArgs& a, size_t row0,
                                           int c0, int nt, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const int cq = lane & 31, hf = lane >> 5;
  const bf16* q = static_cast<const bf16*>(a.q);
  const bf16* k = static_cast<const bf16*>(a.k);
  const bf16* v = static_cast<const bf16*>(a.v);
  constexpr int DV = 64 * NT;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int t = 16 * wave + 8 * hf + u;
    const size_t row = row0 + c0 + t;
    if (t < nt) {
      r.q[u] = *reinterpret_cast<const bf16x4*>(q + row * kDK + 4 * cq);
      r.k[u] = *reinterpret_cast<const bf16x4*>(k + row * kDK + 4 * cq);
      if (PER_CHANNEL) {
        r.g[u] = *reinterpret_cast<const f32x4*>(a.g + row * kDK + 4 * cq);
      } else {
        const float gg = a.g[row];
        r.g[u] = f32x4{gg, gg, gg, gg};
      }
    } else {
      r.q[u] = pack4(0.f, 0.f, 0.f, 0.f);
      r.k[u] = r.q[u];
      r.g[u] = zero4();
    }
  }
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int seg = tid + kThreads * i;
    const int t = seg / (DV / 8), c8 = seg % (DV / 8);
    if (t < nt) {
      r.v[i] = *reinterpret_cast<const bf16x8*>(v + (row0 + c0 + t) * DV + 8 * c8);
    } else {
      const bf16x4 z = pack4(0.f, 0.f, 0.f, 0.f);
      r.v[i] = cat8(z, z);
    }
  }
  r.beta = (tid < kC && tid < nt) ? a.beta[row0 + c0 + tid] : 0.f;
}

template <int NT, bool PER_CHANNEL>
__global__ __launch_bounds__(kThreads) void chunk_mfma_kernel(ChunkArgs a) {
  __shared__ __align__(16) Smem sm;
  constexpr int DV = 64 * NT;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int cq = lane & 31, hf = lane >> 5;  // decay phase: 4 channels, half sub-block
  const int rr = lane & 15, p = lane >> 4;   // matrix-core phases

  const int chain = blockIdx.x;
  const int n = chain / a.H;
  const int h = chain % a.H;
  const TokenRange tr = token_range(a.cu, n, a.T);
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0;
  const size_t state_off = ((size_t)n * a.H + h) * kDK * DV;

  // state S[channel][column] for this wavefront's NT column tiles, accumulator layout:
  // S_acc[n][m][e] = S[16 m + 4 p + e][16 (wave NT + n) + rr]
  f32x4 S_acc[NT][8];
#pragma unroll
  for (int nn = 0; nn < NT; ++nn) {
    const int col = 16 * (wave * NT + nn) + rr;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S_acc[nn][m][e] = a.s0 ? a.s0[state_off + (size_t)(16 * m + 4 * p + e) * DV + col] : 0.f;
      }
    }
  }

  ChunkRegs<NT> cur;
  if (tr.len > 0) load_chunk<NT, PER_CHANNEL>(cur, a, row0, 0, min(kC, tr.len), tid);

  for (int c0 = 0; c0 < tr.len; c0 += kC) {
    const int nt = min(kC, tr.len - c0);
    lds_barrier();  // the previous chunk's state pass is done with LDS

    // ---- decay products inside sub-block I = wave, tokens 8 hf + u, channels 4 cq + j:
    //      P = exp(G_t - R_I) (inclusive prefix), E = exp(R_{I+1} - G_t) (exclusive suffix)
    f32x4 P[8], E[8];
    {
      f32x4 run = {1.f, 1.f, 1.f, 1.f};
      f32x4 al[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          al[u][j] = __expf(cur.g[u][j]);
          run[j] *= al[u][j];
        }
        P[u] = run;
      }
      const f32x4 half_tot = run;
      f32x4 rs = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int u = 7; u >= 0; --u) {
        E[u] = rs;
#pragma unroll
        for (int j = 0; j < 4; ++j) rs[j] *= al[u][j];
      }
      f32x4 other;
#pragma unroll
      for (int j = 0; j < 4; ++j) other[j] = __shfl_xor(half_tot[j], 32, 64);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (hf) P[u][j] *= other[j];   // upper half: times the lower half's product
          else E[u][j] *= other[j];      // lower half: times the upper half's product
        }
      }
      if (hf == 0) {
        f32x4 t4;
#pragma unroll
        for (int j = 0; j < 4; ++j) t4[j] = half_tot[j] * other[j];
        *reinterpret_cast<f32x4*>(&sm.tot[wave][4 * cq]) = t4;
      }
      if (tid < kC) sm.beta[tid] = cur.beta;
    }
    lds_barrier();

    // ---- operands of the A tiles (to LDS) and of the state pass (kept packed in registers)
    bf16x4 qh_r[8], kh_r[8];
    bf16x8 kdec_r[4];
    {
      f32x4 tt[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) tt[I] = *reinterpret_cast<const f32x4*>(&sm.tot[I][4 * cq]);
      f32x4 eR, tail, rtot, far1, far2, far12;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float er = 1.f, tl = 1.f;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (I < wave) er *= tt[I][j];
          if (I > wave) tl *= tt[I][j];
        }
        eR[j] = er;
        tail[j] = tl;
        rtot[j] = 1.f / tt[wave][j];
        far1[j] = tt[1][j];
        far2[j] = tt[2][j];
        far12[j] = tt[1][j] * tt[2][j];
      }
      if (wave == 0 && hf == 0) {
        f32x4 eg;
#pragma unroll
        for (int j = 0; j < 4; ++j) eg[j] = tt[0][j] * tt[1][j] * tt[2][j] * tt[3][j];
        *reinterpret_cast<f32x4*>(&sm.egc[4 * cq]) = eg;
      }
      float kdec_f[4][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = 16 * wave + 8 * hf + u;
        f32x4 qr, kr, kc, kd, qh, kh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float qv = static_cast<float>(cur.q[u][j]);
          const float kv = static_cast<float>(cur.k[u][j]);
          qr[j] = qv * P[u][j];
          kr[j] = kv * P[u][j];
          kc[j] = kv * E[u][j];
          kd[j] = kc[j] * rtot[j];
          qh[j] = qr[j] * eR[j];
          kh[j] = kr[j] * eR[j];
          kdec_f[j][u] = kc[j] * tail[j];
        }
        qh_r[u] = pack4(qh);
        kh_r[u] = pack4(kh);
        st4(&sm.x.a.qr[t][4 * cq], qr);
        st4(&sm.x.a.kr[t][4 * cq], kr);
        st4(&sm.x.a.kd[t][4 * cq], kd);
        if (wave < 3) st4(&sm.x.a.kc[t][4 * cq], kc);
        if (wave == 0) {
          f32x4 f1, f12;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f1[j] = kc[j] * far1[j];
            f12[j] = kc[j] * far12[j];
          }
          st4(&sm.x.a.kfar[t][4 * cq], f1);
          st4(&sm.x.a.kfar[32 + t][4 * cq], f12);
        } else if (wave == 1) {
          f32x4 f2;
#pragma unroll
          for (int j = 0; j < 4; ++j) f2[j] = kc[j] * far2[j];
          st4(&sm.x.a.kfar[t][4 * cq], f2);  // rows 16..31
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int u = 0; u < 8; ++u) kdec_r[j][u] = static_cast<bf16>(kdec_f[j][u]);
      }
    }
    lds_barrier();

    // ---- A_qk and A_kk tiles: tile tau = wave, wave + 4, wave + 8 of the 10 (I, J), J <= I
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int tau = wave + 4 * s;
      if (tau < 10) {
        const int I = tau >= 6 ? 3 : tau >= 3 ? 2 : tau >= 1 ? 1 : 0;
        const int J = tau - I * (I + 1) / 2;
        const bf16* col;
        if (J == I) col = &sm.x.a.kd[16 * J][0];
        else if (J == I - 1) col = &sm.x.a.kc[16 * J][0];
        else if (I == 2) col = &sm.x.a.kfar[0][0];        // (2, 0)
        else if (J == 1) col = &sm.x.a.kfar[16][0];       // (3, 1)
        else col = &sm.x.a.kfar[32][0];                   // (3, 0)
        f32x4 accq = zero4(), acck = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int ch = 32 * ks + 8 * p;
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(col + rr * kLDK + ch);
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.x.a.qr[16 * I + rr][ch]);
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&sm.x.a.kr[16 * I + rr][ch]);
          accq = mfma32(aq, b, accq);
          acck = mfma32(ak, b, acck);
        }
        const int j = 16 * J + rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * I + 4 * p + e;
          const bool lower_q = J < I || j <= i;
          const bool lower_k = J < I || j < i;
          const float vq = lower_q ? accq[e] : 0.f;
          const float vk = lower_k ? sm.beta[i] * acck[e] : 0.f;
          sm.aqk[i][j] = static_cast<bf16>(vq);
          sm.akk_neg[i][j] = static_cast<bf16>(-vk);
          if (J == I) sm.adiag[I][4 * p + e][rr] = vk;
        }
      }
    }
    lds_barrier();

    // ---- diagonal inverses (one 16 x 16 block per wavefront, one column per lane) and
    //      the state-pass operands (written over the A-tile operands, now dead)
    if (lane < 16) {
      float x[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        float s = m == lane ? 1.f : 0.f;
#pragma unroll
        for (int kk = 0; kk < m; ++kk) s -= sm.adiag[wave][m][kk] * x[kk];
        x[m] = s;
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) sm.tdiag[wave][m][lane] = static_cast<bf16>(x[m]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = 16 * wave + 8 * hf + u;
      *reinterpret_cast<bf16x4*>(&sm.x.s.qh[t][4 * cq]) = qh_r[u];
      *reinterpret_cast<bf16x4*>(&sm.x.s.kh[t][4 * cq]) = kh_r[u];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<bf16x8*>(&sm.x.s.kdecT[4 * cq + j][16 * wave + 8 * hf]) = kdec_r[j];
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const int seg = tid + kThreads * i;
      const int t = seg / (DV / 8), c8 = seg % (DV / 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.x.s.vT[8 * c8 + j][t] = cur.v[i][j];
    }
    lds_barrier();

    // every input of this chunk is in LDS now: fetch the next chunk while computing
    if (c0 + kC < tr.len)
      load_chunk<NT, PER_CHANNEL>(cur, a, row0, c0 + kC, min(kC, tr.len - c0 - kC), tid);

    // ---- state pass for this wavefront's NT column tiles
    // B operands of S (bf16), contraction permuted over channels
    bf16x8 sb[NT][4];
#pragma unroll
    for (int nn = 0; nn < NT; ++nn)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sb[nn][ks] = cat8(pack4(S_acc[nn][2 * ks]), pack4(S_acc[nn][2 * ks + 1]));

    bf16x4 vp[NT][4];  // V' per sub-block, bf16, accumulator layout = 16x16x16 B layout
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 X[NT], Oi[NT];
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) {
        X[nn] = zero4();
        Oi[nn] = zero4();
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16* kr_ = &sm.x.s.kh[16 * I + rr][32 * ks + 4 * p];
        const bf16* qr_ = &sm.x.s.qh[16 * I + rr][32 * ks + 4 * p];
        const bf16x8 ak = cat8(*reinterpret_cast<const bf16x4*>(kr_),
                               *reinterpret_cast<const bf16x4*>(kr_ + 16));
        const bf16x8 aq = cat8(*reinterpret_cast<const bf16x4*>(qr_),
                               *reinterpret_cast<const bf16x4*>(qr_ + 16));
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) {
          X[nn] = mfma32(ak, sb[nn][ks], X[nn]);
          Oi[nn] = mfma32(aq, sb[nn][ks], Oi[nn]);
        }
      }
      // B_I = beta (V - K^ S), then V'_I = T_II (B_I - sum_{J<I} A_kk[I,J] V'_J)
      f32x4 bt;
#pragma unroll
      for (int e = 0; e < 4; ++e) bt[e] = sm.beta[16 * I + 4 * p + e];
      const bf16x4 tI = *reinterpret_cast<const bf16x4*>(&sm.tdiag[I][rr][4 * p]);
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) {
        const int col = 16 * (wave * NT + nn) + rr;
        const bf16x4 vv = *reinterpret_cast<const bf16x4*>(&sm.x.s.vT[col][16 * I + 4 * p]);
        f32x4 R;
#pragma unroll
        for (int e = 0; e < 4; ++e) R[e] = bt[e] * (static_cast<float>(vv[e]) - X[nn][e]);
#pragma unroll
        for (int J = 0; J < I; ++J) {
          const bf16x4 aij =
              *reinterpret_cast<const bf16x4*>(&sm.akk_neg[16 * I + rr][16 * J + 4 * p]);
          R = mfma16(aij, vp[nn][J], R);
        }
        const f32x4 vI = mfma16(tI, pack4(R), zero4());
        vp[nn][I] = pack4(vI);
      }
      // O_I = Q^_I S + sum_{J<=I} A_qk[I, J] V'_J
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const bf16x4 aij = *reinterpret_cast<const bf16x4*>(&sm.aqk[16 * I + rr][16 * J + 4 * p]);
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) Oi[nn] = mfma16(aij, vp[nn][J], Oi[nn]);
      }
      bf16* o = static_cast<bf16*>(a.o);
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) {
        const int col = 16 * (wave * NT + nn) + rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + 4 * p + e;
          if (t < nt) o[(row0 + c0 + t) * DV + col] = static_cast<bf16>(Oi[nn][e]);
        }
      }
    }

    // S <- Diag(exp G_C) S + K_dec^T V'
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const f32x4 eg = *reinterpret_cast<const f32x4*>(&sm.egc[16 * m + 4 * p]);
      const bf16* kd_ = &sm.x.s.kdecT[16 * m + rr][4 * p];
      const bf16x8 a0 = cat8(*reinterpret_cast<const bf16x4*>(kd_),
                             *reinterpret_cast<const bf16x4*>(kd_ + 16));
      const bf16x8 a1 = cat8(*reinterpret_cast<const bf16x4*>(kd_ + 32),
                             *reinterpret_cast<const bf16x4*>(kd_ + 48));
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) {
        f32x4 s = S_acc[nn][m];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] *= eg[e];
        s = mfma32(a0, cat8(vp[nn][0], vp[nn][1]), s);
        s = mfma32(a1, cat8(vp[nn][2], vp[nn][3]), s);
        S_acc[nn][m] = s;
      }
    }
  }

  if (a.sT) {
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) {
      const int col = 16 * (wave * NT + nn) + rr;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.sT[state_off + (size_t)(16 * m + 4 * p + e) * DV + col] = S_acc[nn][m][e];
    }
  }
}

template <int NT, bool PER_CHANNEL>
hipError_t launch_nt(const ChunkArgs& a, hipStream_t stream) {
  chunk_mfma_kernel<NT, PER_CHANNEL><<<dim3(a.N * a.H), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supports(int dk, int dv) { return dk == kDK && (dv == 64 || dv == 128); }

hipError_t launch_chunk_mfma(const ChunkArgs& a, bool per_channel, hipStream_t stream) {
  if (!chunk_mfma_supports(a.dk, a.dv)) return hipErrorInvalidValue;
  if (a.dv == 128)
    return per_channel ? launch_nt<2, true>(a, stream) : launch_nt<2, false>(a, stream);
  return per_channel ? launch_nt<1, true>(a, stream) : launch_nt<1, false>(a, stream);
}

}  // namespace kda
