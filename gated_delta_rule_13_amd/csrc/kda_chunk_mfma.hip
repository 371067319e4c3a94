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
// Layout: one workgroup per chain (sequence, head) with eight wavefronts in two roles.
// The four "prep" wavefronts each own one 16-token block of the next 64 tokens: they
// load its q, k, g, beta, compute the decay products and the bf16 operands into LDS, then
// the block's A_qk / A_kk tile and the inverse of its (I + Diag(beta) A_kk) on the fp32
// matrix cores -- no other wavefront is involved, so they need no barrier. The four
// "state" wavefronts each own dv / 4 value columns of the state for the whole sequence,
// held in matrix-core accumulator registers, and run the four blocks' state steps of the
// current 64 tokens from the other LDS buffer; their outputs go through an LDS tile and
// leave as 16-byte pieces of token rows. One workgroup barrier per 64 tokens swaps the
// two buffers, so the vector-ALU work of preparing tokens t + 64 overlaps the
// matrix-core chain of the state steps of tokens t.
//
// Matrix-core operand layouts used (lane l, r = l % 16, p = l / 16):
//   16x16x32 bf16: A[r][8p + i], B[8p + i][r] (i < 8); D[4p + e][r] (e < 4)
//   16x16x16 bf16: A[r][4p + i], B[4p + i][r] (i < 4); D[4p + e][r]
//   16x16x4  fp32: A[r][p], B[p][r]; D[4p + e][r]
// The D layout of one product is the B layout of a 16x16x16 product, which chains the
// UT solve and the state update in registers. A state wavefront keeps its dk x 16 slice of
// S as eight accumulator tiles whose rows are a fixed permutation of the key channels:
// tile m = 2 s + h, row 4 p + e holds channel 32 s + 8 p + 4 h + e. Then tiles 2 s and
// 2 s + 1 together are the B operand of a 16x16x32 product over channels [32 s, 32 s + 32)
// in natural order, and the matching A operand is 16 contiguous bytes of a token row.
//
// Global memory is read and written through buffer descriptors bounded by the chain's
// rows: reads past the sequence's end return zero (q = k = 0, g = 0, beta = 0 is the
// identity token) and writes past it are dropped, so partial chunks need no branches.
#include <stddef.h>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace {


constexpr int kC = 64;         // tokens prepared and consumed per step (four blocks)
constexpr int kLDK = kDK + 8;  // padded LDS row (bf16) of [token][channel] tiles
constexpr int kLDT = kC + 8;   // padded LDS row (bf16) of [channel][token] tiles
constexpr int kPrepWaves = 4;  // one per 16-token block
constexpr int kModeOut = 0, kModeHist = 1, kModeState = 2, kModeTrans = 3;  // see state_role
constexpr int kModePair = 4;  // launch of both kModeState and kModeTrans items (see the kernel)

#ifndef KDA_STATE_PRIO
#define KDA_STATE_PRIO 3
#endif


// Operands of 64 tokens, written by the prep wavefronts and read by the state wavefronts.
struct Stage {
  bf16 qr[kC][kLDK];      // q * P
  bf16 kr[kC][kLDK];      // k * P
  bf16 kcT[kDK][kLDT];    // (k * E)^T
  bf16 aqk[4][16][24];    // A_qk of each block (lower, diagonal included)
  bf16 tdiag[4][16][24];  // (I + Diag(beta) A_kk)^-1 of each block
  float tot[4][kDK];      // decay over each block
  float beta[kC];
};
struct Smem {
  Stage st[2];            // double buffer
  bf16 kd[kC][kLDK];      // k / P (prep wavefronts only; each reads back its own rows)
  bf16 ost[kC][kLDK];     // outputs of the last 64 tokens (each state wavefront: its columns)
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget of one CU");
static_assert(sizeof(Stage) % 16 == 0 && offsetof(Stage, kcT) % 16 == 0 &&
                  offsetof(Stage, aqk) % 16 == 0 && offsetof(Stage, tdiag) % 16 == 0 &&
                  offsetof(Stage, tot) % 16 == 0 && offsetof(Smem, kd) % 16 == 0 &&
                  offsetof(Smem, ost) % 16 == 0,
              "vector LDS accesses need 16-byte aligned arrays");
static_assert((kLDK * 2) % 16 == 0 && (kLDT * 2) % 16 == 0, "row pitch must keep alignment");



// Decay products of block I and its bf16 operands, written to LDS by one wavefront:
// alpha = exp(g); P_t = exp(G_t - G_0) is the inclusive prefix product of alpha, E_t =
// exp(G_16 - G_t) the product after t, tot = exp(G_16 - G_0), and k / P_t = k E_t / tot.
// A lane holds 8 tokens of one half block; the halves exchange their products.
// For Gated Delta Rule-2 the read-side operand is (b * k) P, b the erase gate: it serves
// both the prediction (b * k)^T S and the strictly lower (b * k) (k / P)^T of the solve.
template <bool GDR2>
__device__ __forceinline__ void prep_block(Stage& st, bf16 (*kd)[kLDK], const BlockRegs& r,
                                           int I, int lane) {
  const int cq = lane & 31, hf = lane >> 5;
  f32x4 al[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) al[u][j] = __expf(r.g[u][j]);
  f32x4 half = al[0];
#pragma unroll
  for (int u = 1; u < 8; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) half[j] *= al[u][j];
  f32x4 tot, rtot, run, rs;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float other = __shfl_xor(half[j], 32, 64);  // the other half block's product
    tot[j] = half[j] * other;
    rtot[j] = __builtin_amdgcn_rcpf(tot[j]);
    run[j] = hf ? other : 1.f;  // prefix entering this half
    rs[j] = hf ? 1.f : other;   // product after this half
  }
  if (hf == 0) *reinterpret_cast<f32x4*>(&st.tot[I][4 * cq]) = tot;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int t = 16 * I + 8 * hf + u;
    f32x4 qr, kr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      run[j] *= al[u][j];
      qr[j] = static_cast<float>(r.q[u][j]) * run[j];
      kr[j] = static_cast<float>(r.k[u][j]) * (GDR2 ? r.b[u][j] * run[j] : run[j]);
    }
    *reinterpret_cast<bf16x4*>(&st.qr[t][4 * cq]) = pack4(qr);
    *reinterpret_cast<bf16x4*>(&st.kr[t][4 * cq]) = pack4(kr);
  }
#pragma unroll
  for (int h4 = 1; h4 >= 0; --h4) {
    float kcv[4][4];
#pragma unroll
    for (int uu = 3; uu >= 0; --uu) {
      const int u = 4 * h4 + uu;
      const int t = 16 * I + 8 * hf + u;
      f32x4 kdv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kcv[j][uu] = static_cast<float>(r.k[u][j]) * rs[j];
        kdv[j] = kcv[j][uu] * rtot[j];
        rs[j] *= al[u][j];
      }
      *reinterpret_cast<bf16x4*>(&kd[t][4 * cq]) = pack4(kdv);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<bf16x4*>(&st.kcT[4 * cq + j][16 * I + 8 * hf + 4 * h4]) =
          pack4(kcv[j][0], kcv[j][1], kcv[j][2], kcv[j][3]);
  }
  if (lane < 16) st.beta[16 * I + lane] = r.beta;
}


// The A_qk / A_kk tile of block I and the inverse of its (I + N), N = Diag(beta) A_kk
// strictly lower (unit_lower_inverse).
__device__ __forceinline__ void block_tiles(Stage& st, const bf16 (*kd)[kLDK], int I, int rr,
                                            int p) {
  bf16x8 bq[4], bk[4], bc[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = 32 * ks + 8 * p;
    bq[ks] = *reinterpret_cast<const bf16x8*>(&st.qr[16 * I + rr][ch]);
    bk[ks] = *reinterpret_cast<const bf16x8*>(&st.kr[16 * I + rr][ch]);
    bc[ks] = *reinterpret_cast<const bf16x8*>(&kd[16 * I + rr][ch]);
  }
  f32x4 accq = zero4(), acck = zero4(), acct = zero4();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    accq = mfma32(bq[ks], bc[ks], accq);   // A_qk[i][j], lane holds i = 4p + e, j = rr
    acck = mfma32(bk[ks], bc[ks], acck);   // A_kk[i][j]
    acct = mfma32(bc[ks], bk[ks], acct);   // A_kk[j][i]: lane holds A_kk[rr][4p + e]
  }
  f32x4 nc, nr;
  const float brr = st.beta[16 * I + rr];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * p + e;
    st.aqk[I][i][rr] = static_cast<bf16>(rr <= i ? accq[e] : 0.f);
    nc[e] = rr < i ? st.beta[16 * I + i] * acck[e] : 0.f;   // N[i][rr]
    nr[e] = i < rr ? brr * acct[e] : 0.f;                    // N[rr][i]
  }
  const f32x4 inv = unit_lower_inverse(nc, nr, rr, p);
#pragma unroll
  for (int e = 0; e < 4; ++e) st.tdiag[I][4 * p + e][rr] = static_cast<bf16>(inv[e]);
}

// Values of one state column for the 16 tokens of block I, in the accumulator layout
// (token 16 I + 4 p + e), kept as raw bf16 so that nothing waits for the loads before the
// step that uses them. off is the byte offset of token 16 I + 4 p in this column.
template <int DV>
__device__ __forceinline__ void load_values(bf16 (&vv)[4], rsrc_t v, uint32_t off) {
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = ld_b16(v, off + e * DV * 2);
}

// Write gates of one value column for the 16 tokens of block I (fp32, same layout as
// load_values; off is the byte offset of token 16 I + 4 p in this column of the gates).
template <int DV>
__device__ __forceinline__ void load_gates(float (&ww)[4], rsrc_t w, uint32_t off) {
#pragma unroll
  for (int e = 0; e < 4; ++e) ww[e] = ld_b32(w, off + e * DV * 4);
}

// Stores the outputs of chunk `step` that this state wavefront staged in LDS (its 16 nt
// columns from cbase, 64 token rows) as 16-byte row pieces; rows past the chain are dropped.
template <int DV>
__device__ __forceinline__ void flush_outputs(const Smem& sm, rsrc_t odst, int step, int cbase,
                                              int nt, int lane) {
  for (int i = 0; i < 2 * nt; ++i) {
    const int idx = lane + 64 * i;
    const int t = idx / (2 * nt);
    const int c0 = cbase + 8 * (idx % (2 * nt));
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(&sm.ost[t][c0]);
    st_b128(odst, (uint32_t)((step * kC + t) * DV + c0) * 2, x);
  }
}

// State wavefront: NT 16-column tiles of S starting at column cbase, for the whole chain.
// Whole chains use the kernel's tile count, half items half of it; each is its own
// straight-line instantiation (a tile count chosen at run time inside the loops would let
// branches remove instructions that the wait states after the matrix-core products were
// counted on).
// MODE selects what the wavefront produces besides the final state (written to sTp, the
// dk x dv row-major matrix of this item, when not null; s0p likewise for the initial state):
//   kModeOut   the outputs o (the forward itself);
//   kModeHist  the state at every block start in a.hist (at byte hist_off, the layout of
//              hist_chain_offset), for the backward pass; no outputs;
//   kModeState nothing else (the end state of a segment started from zero);
//   kModeTrans the transition of the segment: the identity as initial state and zero values,
//              so that the final state is the dk x dk product of the segment's token maps.
template <int NT, int DV, bool GDR2, int MODE>
__device__ __forceinline__ void state_role(Smem& sm, const ChunkArgs& a, const TokenRange& tr,
                                           size_t row0, const float* s0p, float* sTp,
                                           size_t hist_off, int nsteps, int cbase, int lane,
                                           int rr, int p) {
  constexpr bool HIST = MODE == kModeHist, OUT = MODE == kModeOut, TRANS = MODE == kModeTrans;
  // (the transition reads no values: a zero-sized view returns zeros)
  const rsrc_t vsrc = make_rsrc(static_cast<const bf16*>(a.v) + row0 * DV,
                                TRANS ? 0u : (uint32_t)tr.len * DV * 2);
  const rsrc_t odst = make_rsrc(static_cast<bf16*>(a.o) + row0 * DV, (uint32_t)tr.len * DV * 2);
  const rsrc_t hdst = make_rsrc(static_cast<char*>(a.hist) + (HIST ? hist_off : 0),
                                HIST ? (uint32_t)nsteps * 4 * kDK * DV * 2 : 0);
  int col[NT];
  uint32_t voff[NT];  // byte offset of (token 4 p, column col) within a 64-token chunk
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    col[c] = cbase + 16 * c + rr;
    voff[c] = (uint32_t)(4 * p * DV + col[c]) * 2;
  }
  // S_acc[c][m][e] = S[32 (m / 2) + 8 p + 4 (m % 2) + e][col[c]]
  f32x4 S_acc[NT][8];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 32 * (m >> 1) + 8 * p + 4 * (m & 1) + e;
        S_acc[c][m][e] = TRANS ? (ch == col[c] ? 1.f : 0.f)
                               : (s0p ? s0p[(size_t)ch * DV + col[c]] : 0.f);
      }
  bf16 vv[NT][4][4];
  float ww[NT][4][4];  // write gate of the values (Gated Delta Rule-2 only)
  const rsrc_t wsrc = GDR2 ? make_rsrc(a.write + row0 * DV, (uint32_t)tr.len * DV * 4) : vsrc;
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      load_values<DV>(vv[c][I], vsrc, voff[c] + I * 16 * DV * 2);
      if (GDR2) load_gates<DV>(ww[c][I], wsrc, 2 * (voff[c] + I * 16 * DV * 2));
    }
  // the initial state must be in registers before the loop, or the loop would wait
  // for these loads on every pass
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  lds_barrier();
  for (int s = 0; s < nsteps; ++s) {
    const Stage& st = sm.st[s & 1];
    const uint32_t cbyte = (uint32_t)s * kC * DV * 2;
    // the barrier ending the previous step waited for this wavefront's staging writes
    if (OUT && s > 0) flush_outputs<DV>(sm, odst, s - 1, cbase, NT, lane);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      // X = (K P) S, S as the B operand (bf16), and O^T = S^T (Q P)^T, S^T as the A
      // operand (the same registers): O^T leaves each lane with four consecutive
      // columns of one token
      f32x4 X[NT], Ot[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) X[c] = Ot[c] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&st.kr[16 * I + rr][32 * ks + 8 * p]);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const bf16x8 sb = cat8(pack4(S_acc[c][2 * ks]), pack4(S_acc[c][2 * ks + 1]));
          X[c] = mfma32(ak, sb, X[c]);
          if constexpr (HIST) {
            const uint32_t tile = (uint32_t)(4 * s + I) * (DV / 16) + (cbase + 16 * c) / 16;
            st_b128(hdst, ((tile * 4 + ks) * 64 + lane) * 16, sb);
          } else if constexpr (OUT) {
            const bf16x8 aq =
                *reinterpret_cast<const bf16x8*>(&st.qr[16 * I + rr][32 * ks + 8 * p]);
            Ot[c] = mfma32(sb, aq, Ot[c]);
          }
        }
      }
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&st.beta[16 * I + 4 * p]);
      const bf16x4 tI = *reinterpret_cast<const bf16x4*>(&st.tdiag[I][rr][4 * p]);
      const bf16x4 aI = *reinterpret_cast<const bf16x4*>(&st.aqk[I][rr][4 * p]);
      // V' = Tm Diag(beta) (V - X)
      bf16x4 vp[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        f32x4 R;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          R[e] = GDR2 ? ww[c][I][e] * static_cast<float>(vv[c][I][e]) - X[c][e]
                      : bt[e] * (static_cast<float>(vv[c][I][e]) - X[c][e]);
        vp[c] = pack4(R);
        // the next 64 tokens' values of this block
        load_values<DV>(vv[c][I], vsrc, voff[c] + cbyte + (I * 16 + kC) * DV * 2);
        if (GDR2) load_gates<DV>(ww[c][I], wsrc, 2 * (voff[c] + cbyte + (I * 16 + kC) * DV * 2));
      }
#pragma unroll
      for (int c = 0; c < NT; ++c) vp[c] = pack4(mfma16(tI, vp[c], zero4()));
      // O^T += V'^T A_qk^T, staged as bf16 token rows. The product starts from zero
      // and O^T is added on the vector ALU: accumulating a 16x16x16 product onto the
      // result of a 16x16x32 product still in flight delays its completion beyond the
      // wait states counted from its issue, and the conversion below then read stale
      // registers.
      if constexpr (OUT) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const bf16x4 ob = pack4(Ot[c] + mfma16(vp[c], aI, zero4()));
          *reinterpret_cast<bf16x4*>(&sm.ost[16 * I + rr][cbase + 16 * c + 4 * p]) = ob;
        }
      }
      // S <- Diag(tot) S + (K E)^T V'
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int s2 = m >> 1, h2 = m & 1;
        // tot of this lane's rows: one float per lane, spread over its quad
        const float d1 = st.tot[I][32 * s2 + 8 * p + 4 * h2 + (rr & 3)];
        const int cha = 32 * s2 + 8 * (rr >> 2) + 4 * h2 + (rr & 3);  // channel of A row rr
        const bf16x4 ac = *reinterpret_cast<const bf16x4*>(&st.kcT[cha][16 * I + 4 * p]);
        const f32x4 dc = {quad_bcast<0>(d1), quad_bcast<1>(d1), quad_bcast<2>(d1),
                          quad_bcast<3>(d1)};
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          f32x4 s_ = S_acc[c][m];
#pragma unroll
          for (int e = 0; e < 4; ++e) s_[e] *= dc[e];
          S_acc[c][m] = mfma16(ac, vp[c], s_);
        }
      }
    }
    lds_barrier();
  }
  if (OUT && nsteps > 0) flush_outputs<DV>(sm, odst, nsteps - 1, cbase, NT, lane);
  if (sTp) {
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ch = 32 * (m >> 1) + 8 * p + 4 * (m & 1) + e;
          sTp[(size_t)ch * DV + col[c]] = S_acc[c][m][e];
        }
  }
}

template <int NS, int NT, bool PER_CHANNEL, bool GDR2, int MODE>
__global__ __launch_bounds__(64 * (kPrepWaves + NS)) void chunk_mfma_kernel(ChunkArgs a) {
  constexpr bool HIST = MODE == kModeHist;
  constexpr int DV = 16 * NS * NT;
  __shared__ __align__(16) Smem sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int rr = lane & 15, p = lane >> 4;
  const bool prep_wave = wave < kPrepWaves;

  // work item: a chain, or one half of its value columns
  int chain = blockIdx.x, part = 0;
  if (a.plan) {
    if (blockIdx.x >= a.plan[0]) return;  // the grid is sized for the largest schedule
    const uint32_t item = a.plan[1 + blockIdx.x];
    chain = (int)(item >> 2);
    part = (int)(item & 3);
  } else if (NT > 1 && a.split_all) {
    uint32_t c, pt;
    split_item(blockIdx.x, (uint32_t)(a.N * a.H * (a.seg_len > 0 ? a.nseg : 1)), c, pt);
    chain = (int)c;
    part = (int)pt;
  }
  // kModePair: even items compute segment end states, odd items their transitions (the
  // transitions in a.hist as fp32 dk x dk matrices; DV = dk)
  int kind = MODE;
  if constexpr (MODE == kModePair) {
    kind = chain & 1 ? kModeTrans : kModeState;
    chain >>= 1;
  }
  // with segments, an item is segment `seg` of its chain (segments of seg_len tokens)
  int seg = 0;
  if (a.seg_len > 0) {
    seg = chain % a.nseg;
    chain /= a.nseg;
  }
  const int n = chain / a.H;
  const int h = chain % a.H;
  TokenRange tr = token_range(a.cu, n, a.T);
  const size_t mat = (size_t)n * a.H + h;  // the chain's state matrix
  const float* s0p = a.s0 ? a.s0 + mat * kDK * DV : nullptr;
  float* sTp = a.sT ? a.sT + mat * kDK * DV : nullptr;
  if (a.seg_len > 0) {
    const int nseg_n = tr.len > 0 ? (tr.len + a.seg_len - 1) / a.seg_len : 1;
    // the outputs pass runs every segment; the state and transition passes all but the last
    if (MODE == kModeOut ? seg >= nseg_n : seg >= nseg_n - 1) return;
    const int first = seg * a.seg_len;
    tr.t0 += first;
    tr.len = min(a.seg_len, tr.len - first);
    const size_t item = mat * a.nseg + seg;
    if (MODE == kModeOut) {   // start states of the segments in s0; the chain's in sT
      s0p = a.s0 + item * kDK * DV;
      sTp = (seg == nseg_n - 1 && a.sT) ? a.sT + mat * kDK * DV : nullptr;
    } else {                  // per-segment end states (transitions: dk x dk, DV = dk)
      s0p = nullptr;
      sTp = (kind == kModeTrans && MODE == kModePair ? static_cast<float*>(a.hist) : a.sT) +
            item * kDK * DV;
    }
  }
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0;
  const size_t hist_off = HIST ? hist_chain_offset(a, n, h, tr) : 0;
  const int nsteps = (tr.len + kC - 1) / kC;

  if (prep_wave) {
    // ---------------- prep wavefront: block I of every 64 tokens
    const int I = wave;
    const PrepSrc src = prep_src<PER_CHANNEL, GDR2>(a, row0, tr.len, I, lane);
    BlockRegs r;
    if (nsteps > 0) {
      load_block<PER_CHANNEL, GDR2>(r, src, 0);
      prep_block<GDR2>(sm.st[0], sm.kd, r, I, lane);
      wave_lds_fence();
      block_tiles(sm.st[0], sm.kd, I, rr, p);
      if (nsteps > 1) load_block<PER_CHANNEL, GDR2>(r, src, kC);
    }
    lds_barrier();
    for (int s = 0; s < nsteps; ++s) {
      if (s + 1 < nsteps) {
        Stage& st = sm.st[(s + 1) & 1];
        prep_block<GDR2>(st, sm.kd, r, I, lane);
        wave_lds_fence();
        block_tiles(st, sm.kd, I, rr, p);
        if (s + 2 < nsteps) load_block<PER_CHANNEL, GDR2>(r, src, (s + 2) * kC);
      }
      lds_barrier();
    }
  } else {
    // ---------------- state wavefront
    // The state steps are the sequential critical path; the prep wavefronts sharing a
    // SIMD have slack, so the state wavefronts take issue priority.
    __builtin_amdgcn_s_setprio(KDA_STATE_PRIO);
    const int j = wave - kPrepWaves;
    if constexpr (MODE == kModePair) {  // whole items only
      if (kind == kModeTrans)
        state_role<NT, DV, GDR2, kModeTrans>(sm, a, tr, row0, s0p, sTp, 0, nsteps, 16 * NT * j,
                                             lane, rr, p);
      else
        state_role<NT, DV, GDR2, kModeState>(sm, a, tr, row0, s0p, sTp, 0, nsteps, 16 * NT * j,
                                             lane, rr, p);
      return;
    }
    if constexpr (NT > 1) {
      if (part) {  // a half item: NT / 2 tiles per wavefront over one half of the columns
        state_role<NT / 2, DV, GDR2, MODE>(sm, a, tr, row0, s0p, sTp, hist_off, nsteps,
                                           (part == 2 ? DV / 2 : 0) + 16 * (NT / 2) * j, lane,
                                           rr, p);
        return;
      }
    }
    state_role<NT, DV, GDR2, MODE>(sm, a, tr, row0, s0p, sTp, hist_off, nsteps, 16 * NT * j,
                                   lane, rr, p);
  }
}

// ---------------------------------------------------------------------------------------
// Schedule. With one workgroup per chain the launch lasts as long as the longest chain, and
// packed sequences of very different lengths leave most compute units idle for its second
// half. The scheduler (one workgroup, on the device, so that the call stays asynchronous)
// sorts the sequences by chunk count and splits the value columns of the longest ones over
// two workgroups while that lowers the bound max(longest item, total work / compute units)
// on the makespan; a half item re-does the prep work and half of the state work, costing
// about kHalfCost of the whole chain. Items are listed longest first, which the in-order
// workgroup dispatch turns into longest-processing-time-first list scheduling.

constexpr int kMaxPlanSeqs = 1024;  // sequences one scheduling workgroup sorts

constexpr double kHalfCost = 0.88;  // time of a half-column item relative to its whole chain

__global__ __launch_bounds__(kMaxPlanSeqs) void chunk_plan_kernel(const int32_t* cu, int N, int H,
                                                                  int T, int cus, int allow_split,
                                                                  uint32_t* plan) {
  __shared__ int key[kMaxPlanSeqs];       // chunks of the sequence
  __shared__ int seq[kMaxPlanSeqs];       // sequence index
  __shared__ int ent_seq[kMaxPlanSeqs];   // schedule entries (one per sequence), in order
  __shared__ int ent_parts[kMaxPlanSeqs];
  __shared__ uint32_t ent_off[kMaxPlanSeqs + 1];
  __shared__ int n_ent;
  const int t = threadIdx.x;
  int c = -1;  // padding sorts last
  if (t < N) c = (token_range(cu, t, T).len + kC - 1) / kC;
  key[t] = c;
  seq[t] = t;
  __syncthreads();
  // bitonic sort of the first n2 >= N entries: more chunks first, then lower index
  int n2 = 1;
  while (n2 < N) n2 <<= 1;
  for (int k = 2; k <= n2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int u = t ^ j;
      if (t < n2 && u > t) {
        const bool t_first = key[t] > key[u] || (key[t] == key[u] && seq[t] < seq[u]);
        if (((t & k) == 0) != t_first) {
          const int k0 = key[t], s0 = seq[t];
          key[t] = key[u];
          seq[t] = seq[u];
          key[u] = k0;
          seq[u] = s0;
        }
      }
      __syncthreads();
    }
  if (t == 0) {
    double total = 0.0;  // work in chunk-times of one workgroup
    for (int i = 0; i < N; ++i) total += (double)key[i] * H;
    int ns = 0;  // the ns longest sequences are split
    double maxhalf = 0.0;
    while (allow_split && ns < N && key[ns] > 0) {
      const double c0 = key[ns], next = ns + 1 < N ? key[ns + 1] : 0.0;
      const double bound = fmax(fmax(c0, maxhalf), total / cus);
      const double total2 = total + H * (2.0 * kHalfCost - 1.0) * c0;
      const double maxhalf2 = fmax(maxhalf, kHalfCost * c0);
      if (!(fmax(fmax(next, maxhalf2), total2 / cus) < 0.98 * bound)) break;
      total = total2;
      maxhalf = maxhalf2;
      ++ns;
    }
    // merge split sequences (item cost kHalfCost * chunks) and whole ones by cost
    int a = 0, b = ns, e = 0;
    uint32_t off = 0;
    while (a < ns || b < N) {
      const bool split = a < ns && (b >= N || kHalfCost * key[a] >= key[b]);
      const int i = split ? a++ : b++;
      ent_seq[e] = seq[i];
      ent_parts[e] = split ? 2 : 1;
      ent_off[e] = off;
      off += (uint32_t)H * ent_parts[e];
      ++e;
    }
    ent_off[e] = off;
    n_ent = e;
    plan[0] = off;
  }
  __syncthreads();
  const uint32_t items = ent_off[n_ent];
  for (uint32_t i = t; i < items; i += kMaxPlanSeqs) {
    int lo = 0, hi = n_ent - 1;  // entry holding item i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ent_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const uint32_t local = i - ent_off[lo];
    uint32_t hh = local, part = 0;
    if (ent_parts[lo] == 2) split_item(local, (uint32_t)H, hh, part);
    plan[1 + i] = (((uint32_t)ent_seq[lo] * H + hh) << 2) | part;
  }
}

template <int NS, int NT, bool PER_CHANNEL, int MODE>
hipError_t launch_ns(const ChunkArgs& a, unsigned grid, hipStream_t stream) {
  if constexpr (MODE == kModeOut || MODE == kModeHist) {
    if (a.erase) {
      chunk_mfma_kernel<NS, NT, PER_CHANNEL, true, MODE>
          <<<dim3(grid), dim3(64 * (kPrepWaves + NS)), 0, stream>>>(a);
      return hipGetLastError();
    }
  }
  chunk_mfma_kernel<NS, NT, PER_CHANNEL, false, MODE>
      <<<dim3(grid), dim3(64 * (kPrepWaves + NS)), 0, stream>>>(a);
  return hipGetLastError();
}

// One launch of mode MODE over a.N * a.H chains (times a.nseg segments when a.seg_len > 0):
// value columns split over two workgroups when every half fits on the device at once, or
// the work list of packed sequences (built here) when a.plan is set.
template <int MODE>
hipError_t launch_mode(const ChunkArgs& args, bool per_channel, int dv, hipStream_t stream) {
  ChunkArgs a = args;
  const bool can_split = dv == 128;  // a half of dv = 128 is one 16-column tile per wavefront
  const long long items =
      (long long)a.N * a.H * (a.seg_len > 0 ? a.nseg : 1) * (MODE == kModePair ? 2 : 1);
  unsigned grid = (unsigned)items;
  a.split_all = 0;
  if (a.plan && a.cu && a.seg_len == 0) {
    // packed sequences: the work list is built on the device from cu_seqlens
    chunk_plan_kernel<<<1, kMaxPlanSeqs, 0, stream>>>(a.cu, a.N, a.H, a.T, a.cus, can_split,
                                                      a.plan);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (can_split) grid *= 2;  // the largest schedule; workgroups past its length exit at once
  } else {
    a.plan = nullptr;
    if (MODE != kModePair && can_split && a.cus > 0 && 2 * items <= a.cus) {
      a.split_all = 1;
      grid *= 2;
    }
  }
  // four state wavefronts: two 16-column tiles each for dv = 128, one for dv = 64
  if (dv == 128)
    return per_channel ? launch_ns<4, 2, true, MODE>(a, grid, stream)
                       : launch_ns<4, 2, false, MODE>(a, grid, stream);
  return per_channel ? launch_ns<4, 1, true, MODE>(a, grid, stream)
                     : launch_ns<4, 1, false, MODE>(a, grid, stream);
}

// S_{s+1} = A_s S_s + B_s over the segments of every chain (fp32), from the chain's initial
// state: writes the start state of every segment. One workgroup per (chain, 32 value
// columns); thread (row, half) owns 16 columns of one state row.
__global__ __launch_bounds__(256) void seg_combine_kernel(const int32_t* cu, int N, int H, int T,
                                                          int dv, int seg_len, int nseg,
                                                          const float* s0, const float* Am,
                                                          const float* Bm, float* start) {
  __shared__ float S[kDK][33];
  const int chain = blockIdx.x, cb = 32 * blockIdx.y;
  const int row = threadIdx.x >> 1, c0 = 16 * (threadIdx.x & 1);
  const int len = token_range(cu, chain / H, T).len;
  const int nseg_n = len > 0 ? (len + seg_len - 1) / seg_len : 1;
  const size_t sz = (size_t)kDK * dv;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = s0 ? s0[chain * sz + (size_t)row * dv + cb + c0 + i] : 0.f;
    S[row][c0 + i] = acc[i];
    start[((size_t)chain * nseg) * sz + (size_t)row * dv + cb + c0 + i] = acc[i];
  }
  for (int sg = 0; sg + 1 < nseg_n; ++sg) {
    __syncthreads();
    const size_t item = (size_t)chain * nseg + sg;
    const float* Arow = Am + item * kDK * kDK + (size_t)row * kDK;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = Bm[item * sz + (size_t)row * dv + cb + c0 + i];
    for (int k4 = 0; k4 < kDK; k4 += 4) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(Arow + k4);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += av[kk] * S[k4 + kk][c0 + i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[row][c0 + i] = acc[i];
      start[(item + 1) * sz + (size_t)row * dv + cb + c0 + i] = acc[i];
    }
  }
}

}  // namespace

// Buffer descriptors address at most 2^31 bytes: a chain's g rows (T x dk fp32) must fit.
bool chunk_mfma_supports(int dk, int dv, int T) {
  return dk == kDK && (dv == 64 || dv == 128) && (long long)T * kDK * 4 < (1ll << 31);
}

size_t chunk_plan_bytes(int N, int H, int dv) {
  (void)dv;
  if (N > kMaxPlanSeqs) return 0;  // too many sequences to sort in one workgroup: no schedule
  const size_t words = 1 + 2 * (size_t)N * H;
  return (words * 4 + 255) / 256 * 256;
}

void chunk_seg_config(int N, int H, int T, int dv, int cus, int& seg_len, int& nseg) {
  seg_len = 0;
  nseg = 1;
  if (cus <= 0 || N <= 0 || H <= 0) return;
  // enough segments for about one workgroup per compute unit in the outputs pass (two per
  // chain segment with split value columns), each at least 512 tokens long (measured on the
  // B2 H16 T4096 and B1 H16 T8192 workloads: twice or four times as many segments, or
  // 256-token segments, are slower: the extra rounds of workgroups cost more than the
  // shorter critical path saves)
  constexpr int kSegMinTokens = 512;
  const long long per = (dv == 128 ? 2ll : 1ll) * N * H;
  long long P = cus / per;
  P = P < T / kSegMinTokens ? P : T / kSegMinTokens;
  if (P < 2) return;
  const int L = (int)(((T + P - 1) / P + 63) / 64 * 64);
  seg_len = L;
  nseg = (T + L - 1) / L;
}

size_t chunk_seg_bytes(int N, int H, int T, int dv, int cus) {
  int L, P;
  chunk_seg_config(N, H, T, dv, cus, L, P);
  if (L == 0) return 0;
  // start states and end states (dk x dv) and transitions (dk x dk) of every segment, fp32
  return (size_t)N * H * P * ((size_t)2 * kDK * dv + (size_t)kDK * kDK) * 4;
}

hipError_t launch_chunk_mfma_hist(const ChunkArgs& args, bool per_channel, hipStream_t stream) {
  ChunkArgs a = args;
  if (!a.hist || !chunk_mfma_supports(a.dk, a.dv, a.T)) return hipErrorInvalidValue;
  a.o = nullptr;
  a.seg_len = 0;
  return launch_mode<kModeHist>(a, per_channel, a.dv, stream);  // builds the work list
}

hipError_t launch_chunk_mfma(const ChunkArgs& args, bool per_channel, hipStream_t stream) {
  ChunkArgs a = args;
  if (!chunk_mfma_supports(a.dk, a.dv, a.T)) return hipErrorInvalidValue;
  a.seg_len = 0;
  return launch_mode<kModeOut>(a, per_channel, a.dv, stream);
}

hipError_t launch_chunk_mfma_segmented(const ChunkArgs& args, bool per_channel, void* ws,
                                       hipStream_t stream) {
  ChunkArgs a = args;
  if (!chunk_mfma_supports(a.dk, a.dv, a.T) || a.erase) return hipErrorInvalidValue;
  int L, P;
  chunk_seg_config(a.N, a.H, a.T, a.dv, a.cus, L, P);
  if (L == 0) return hipErrorInvalidValue;
  a.plan = nullptr;
  a.seg_len = L;
  a.nseg = P;
  const size_t items = (size_t)a.N * a.H * P;
  float* start = static_cast<float*>(ws);
  float* Bm = start + items * kDK * a.dv;
  float* Am = Bm + items * kDK * a.dv;
  // 1. end state of every segment but the last, started from zero, and 2. its transition
  // (dk x dk: the identity's dk columns as the state); one launch when dv = dk
  ChunkArgs b = a;
  b.s0 = nullptr;
  b.sT = Bm;
  b.o = nullptr;
  hipError_t e;
  if (a.dv == kDK) {
    b.hist = Am;
    e = launch_mode<kModePair>(b, per_channel, kDK, stream);
    if (e != hipSuccess) return e;
  } else {
    e = launch_mode<kModeState>(b, per_channel, a.dv, stream);
    if (e != hipSuccess) return e;
    b.sT = Am;
    e = launch_mode<kModeTrans>(b, per_channel, kDK, stream);
    if (e != hipSuccess) return e;
  }
  // 3. the start state of every segment
  seg_combine_kernel<<<dim3((unsigned)(a.N * a.H), (unsigned)(a.dv / 32)), 256, 0, stream>>>(
      a.cu, a.N, a.H, a.T, a.dv, L, P, a.s0, Am, Bm, start);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 4. every segment's outputs from its start state; the last one writes the final state
  a.s0 = start;
  return launch_mode<kModeOut>(a, per_channel, a.dv, stream);
}

}  // namespace kda
