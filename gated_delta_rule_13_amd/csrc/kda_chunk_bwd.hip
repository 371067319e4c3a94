// Backward pass of the chunked forward on the CDNA4 matrix cores (bf16 operands, fp32
// accumulate, dk = 128): the gradients of a loss with respect to q, k, v, g, beta and the
// initial state, given its gradients dO with respect to the outputs and dS_T with respect
// to the final state.
//
// The pages give the forward only (their chunkwise-training section states that the
// backward pass has the forward's shapes), so the steps below are the chain rule applied
// to the forward's 16-token block ("Token Mixer I", section "Kimi Delta Attention",
// chunkwise form, with the block of the forward kernel). With S the state entering a block
// and, per key channel, P_t the decay from the block start through token t, E_t the decay
// after t, Gam = P_16, the block computes
//   Qh = q P, Kh = k P, Kb = k / P, Kt = k E,  A = StrictTril(Kh Kb^T), M = Tril(Qh Kb^T),
//   Tm = (I + Diag(beta) A)^-1,  R = V - Kh S,  U = Tm Diag(beta) R,
//   O = Qh S + M U,  S' = Diag(Gam) S + Kt^T U.
// Given dS' (the gradient reaching S') and dO, reverse mode gives
//   dU = M^T dO + Kt dS',  dY = Tm^T dU,  dV = Diag(beta) dY,
//   dS = Diag(Gam) dS' + Qh^T dO - Kh^T Diag(beta) dY                 (the carry)
//   dQh = dO S^T + dM Kb,  dKh = -Diag(beta) dY S^T + dA Kb,  dKb = dA^T Kh + dM^T Qh,
//   dKt = U dS'^T,  with dM = Tril(dO U^T), dA = -StrictTril(Diag(beta) dY U^T),
//   dbeta_t = sum_j dY_tj R_tj - sum_s A_ts (dY U^T)_ts,
//   d log P_t = dQh_t Qh_t + dKh_t Kh_t - dKb_t Kb_t - dKt_t Kt_t   (per channel),
//   d log Gam = sum_t dKt_t Kt_t + Gam * rowsum(dS' * S),
//   dg_s = sum_{t >= s} d log P_t + d log Gam,   dq = dQh P,   dk = dKh P + dKb / P + dKt E.
//
// Three launches:
//   1. the forward state pass with the state history (kda_chunk_mfma.hip): S entering
//      every pair of blocks (the even blocks), bf16, in the layout of hist_chain_offset;
//   2. chunk_bwd_state_kernel: the carry above, one workgroup per chain, from the last
//      block to the first; it records dS' at the end of every pair of blocks (the odd
//      blocks; same layout) and writes dS_0;
//   3. chunk_bwd_grad_kernel: every pair of blocks independently from its (S, dS'), one
//      wavefront per block, the two exchanging the state and the gradient between their
//      blocks: dq, dk, dv, dg, dbeta.
// Launch 2 has the forward's structure: four "prep" wavefronts prepare the operands of
// the next 64 tokens (in reverse) while four "state" wavefronts, holding dS in matrix-core
// accumulators, run the carry of the current 64 tokens; one barrier per 64 tokens.
#include <stddef.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int kC = 64;          // tokens per step (four blocks)
constexpr int kLDK = kDK + 8;   // padded LDS row (bf16) of [token][channel] tiles
constexpr int kLDB = kC + 4;    // padded LDS row (bf16) of [channel][token] tiles (8-byte rows)
constexpr int kPrepWaves = 4;

#ifndef KDA_STATE_PRIO
#define KDA_STATE_PRIO 3
#endif

// ------------------------------------------------------------------ launch 2: the carry

// Operands of 64 tokens for the carry, written by the prep wavefronts.
struct RStage {
  bf16 kc[kC][kLDK];      // Kt = k * E (row-major: A operand of Kt dS')
  bf16 qrT[kDK][kLDB];    // Qh^T (A operand of Qh^T dO)
  bf16 krT[kDK][kLDB];    // Kh^T
  bf16 aqkT[4][16][24];   // M^T of each block
  bf16 tdT[4][16][24];    // Tm^T of each block
  float tot[4][kDK];      // Gam of each block
  float beta[kC];
};
struct RSmem {
  RStage st[2];
  bf16 qg[kC][kLDK];      // Qh / Gam (prep wavefronts only; each reads back its own rows)
  bf16 kg[kC][kLDK];      // Kh / Gam
};
static_assert(sizeof(RSmem) <= 160 * 1024, "LDS budget of one CU");
static_assert(sizeof(RStage) % 16 == 0 && offsetof(RStage, qrT) % 16 == 0 &&
                  offsetof(RStage, krT) % 16 == 0 && offsetof(RStage, aqkT) % 16 == 0 &&
                  offsetof(RStage, tdT) % 16 == 0 && offsetof(RStage, tot) % 16 == 0 &&
                  offsetof(RSmem, qg) % 16 == 0 && offsetof(RSmem, kg) % 16 == 0,
              "vector LDS accesses need aligned arrays");
static_assert((kLDB * 2) % 8 == 0, "transposed rows must keep 8-byte alignment");

// Decay products of block I and its operands for the carry (one wavefront; a lane holds
// 8 tokens x 4 channels as in the forward's prep). With the Gated Delta Rule-2 gates the
// read-side key Kh is (b * k) P and beta is 1 (the write gate acts on the values).
template <bool GDR2>
__device__ __forceinline__ void prep_block_rev(RStage& st, bf16 (*qg)[kLDK], bf16 (*kg)[kLDK],
                                               const BlockRegs& r, int I, int lane) {
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
    const float other = __shfl_xor(half[j], 32, 64);
    tot[j] = half[j] * other;
    rtot[j] = __builtin_amdgcn_rcpf(tot[j]);
    run[j] = hf ? other : 1.f;
    rs[j] = hf ? 1.f : other;
  }
  if (hf == 0) *reinterpret_cast<f32x4*>(&st.tot[I][4 * cq]) = tot;
  float qp[4][8], kp[4][8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int t = 16 * I + 8 * hf + u;
    f32x4 qs, ks;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      run[j] *= al[u][j];
      qp[j][u] = static_cast<float>(r.q[u][j]) * run[j];
      // Gated Delta Rule-2: the read side takes the erase-gated key (b * k) P
      kp[j][u] = static_cast<float>(r.k[u][j]) * (GDR2 ? r.b[u][j] * run[j] : run[j]);
      qs[j] = qp[j][u] * rtot[j];
      ks[j] = kp[j][u] * rtot[j];
    }
    *reinterpret_cast<bf16x4*>(&qg[t][4 * cq]) = pack4(qs);
    *reinterpret_cast<bf16x4*>(&kg[t][4 * cq]) = pack4(ks);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t0 = 16 * I + 8 * hf;
    *reinterpret_cast<bf16x4*>(&st.qrT[4 * cq + j][t0]) =
        pack4(qp[j][0], qp[j][1], qp[j][2], qp[j][3]);
    *reinterpret_cast<bf16x4*>(&st.qrT[4 * cq + j][t0 + 4]) =
        pack4(qp[j][4], qp[j][5], qp[j][6], qp[j][7]);
    *reinterpret_cast<bf16x4*>(&st.krT[4 * cq + j][t0]) =
        pack4(kp[j][0], kp[j][1], kp[j][2], kp[j][3]);
    *reinterpret_cast<bf16x4*>(&st.krT[4 * cq + j][t0 + 4]) =
        pack4(kp[j][4], kp[j][5], kp[j][6], kp[j][7]);
  }
#pragma unroll
  for (int u = 7; u >= 0; --u) {
    const int t = 16 * I + 8 * hf + u;
    f32x4 ke;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ke[j] = static_cast<float>(r.k[u][j]) * rs[j];
      rs[j] *= al[u][j];
    }
    *reinterpret_cast<bf16x4*>(&st.kc[t][4 * cq]) = pack4(ke);
  }
  if (lane < 16) st.beta[16 * I + lane] = r.beta;
}

// M^T and Tm^T of block I: A_qk = (Qh / Gam) Kt^T and A_kk = (Kh / Gam) Kt^T are the
// forward's Qh Kb^T and Kh Kb^T (Kb = Kt / Gam).
__device__ __forceinline__ void block_tiles_rev(RStage& st, const bf16 (*qg)[kLDK],
                                                const bf16 (*kg)[kLDK], int I, int rr, int p) {
  bf16x8 bq[4], bk[4], bc[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = 32 * ks + 8 * p;
    bq[ks] = *reinterpret_cast<const bf16x8*>(&qg[16 * I + rr][ch]);
    bk[ks] = *reinterpret_cast<const bf16x8*>(&kg[16 * I + rr][ch]);
    bc[ks] = *reinterpret_cast<const bf16x8*>(&st.kc[16 * I + rr][ch]);
  }
  f32x4 accq = zero4(), acck = zero4(), acct = zero4();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    accq = mfma32(bq[ks], bc[ks], accq);   // A_qk[4p + e][rr]
    acck = mfma32(bk[ks], bc[ks], acck);   // A_kk[4p + e][rr]
    acct = mfma32(bc[ks], bk[ks], acct);   // A_kk[rr][4p + e]
  }
  f32x4 m, nc, nr;
  const float brr = st.beta[16 * I + rr];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * p + e;
    m[e] = rr <= i ? accq[e] : 0.f;                           // M[i][rr] = M^T[rr][i]
    nc[e] = rr < i ? st.beta[16 * I + i] * acck[e] : 0.f;     // N[i][rr]
    nr[e] = i < rr ? brr * acct[e] : 0.f;                     // N[rr][i]
  }
  *reinterpret_cast<bf16x4*>(&st.aqkT[I][rr][4 * p]) = pack4(m);
  const f32x4 inv = unit_lower_inverse(nc, nr, rr, p);        // Tm[4p + e][rr]
  *reinterpret_cast<bf16x4*>(&st.tdT[I][rr][4 * p]) = pack4(inv);
}

// dO of one value column for the 16 tokens of block I (token 16 I + 4 p + e), raw bf16.
template <int DV>
__device__ __forceinline__ void load_col(bf16x4& x, rsrc_t src, uint32_t off) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = ld_b16(src, off + e * DV * 2);
}

// State wavefront of the carry: NT 16-column tiles of dS from column cbase, whole chain,
// from the last block to the first.
template <int NT, int DV>
__device__ __forceinline__ void carry_role(RSmem& sm, const BwdArgs& b, const TokenRange& tr,
                                           size_t row0, size_t state_off, size_t hist_off,
                                           int nsteps, int cbase, int lane, int rr, int p) {
  const rsrc_t dosrc =
      make_rsrc(static_cast<const bf16*>(b.dout) + row0 * DV, (uint32_t)tr.len * DV * 2);
  const rsrc_t hdst = make_rsrc(static_cast<char*>(b.hist_ds) + hist_off,
                                (uint32_t)nsteps * 2 * kDK * DV * 2);
  int col[NT];
  uint32_t coff[NT];  // byte offset of (token 4 p, column col) within a 64-token step
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    col[c] = cbase + 16 * c + rr;
    coff[c] = (uint32_t)(4 * p * DV + col[c]) * 2;
  }
  // D_acc[c][m][e] = dS[32 (m / 2) + 8 p + 4 (m % 2) + e][col[c]] (the forward's S layout)
  f32x4 D_acc[NT][8];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 32 * (m >> 1) + 8 * p + 4 * (m & 1) + e;
        D_acc[c][m][e] = b.dsT ? b.dsT[state_off + (size_t)ch * DV + col[c]] : 0.f;
      }
  bf16x4 dd[NT][4];
  if (nsteps > 0) {
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int I = 0; I < 4; ++I)
        load_col<DV>(dd[c][I], dosrc, coff[c] + ((nsteps - 1) * kC + 16 * I) * DV * 2);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  lds_barrier();
  for (int s = nsteps - 1; s >= 0; --s) {
    const RStage& st = sm.st[s & 1];
#pragma unroll
    for (int I = 3; I >= 0; --I) {
      const uint32_t blk = 4 * (uint32_t)s + I;
      // dS' of this block (recorded at the end of each pair of blocks), and Kt dS' (dS' as
      // the B operand, bf16)
      f32x4 dU[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) dU[c] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&st.kc[16 * I + rr][32 * ks + 8 * p]);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const bf16x8 db = cat8(pack4(D_acc[c][2 * ks]), pack4(D_acc[c][2 * ks + 1]));
          if (I & 1) {
            const uint32_t tile = (blk / 2) * (DV / 16) + (cbase + 16 * c) / 16;
            st_b128(hdst, ((tile * 4 + ks) * 64 + lane) * 16, db);
          }
          dU[c] = mfma32(ak, db, dU[c]);
        }
      }
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&st.beta[16 * I + 4 * p]);
      const bf16x4 aT = *reinterpret_cast<const bf16x4*>(&st.aqkT[I][rr][4 * p]);
      const bf16x4 tT = *reinterpret_cast<const bf16x4*>(&st.tdT[I][rr][4 * p]);
      bf16x4 dob[NT], nby[NT];
      // the next step's dO of this block (without a branch, which would make the compiler
      // wait for the load there; at s = 0 it reloads this step's, unused)
      const int sn = s > 0 ? s - 1 : 0;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        dob[c] = dd[c][I];
        load_col<DV>(dd[c][I], dosrc, coff[c] + (sn * kC + 16 * I) * DV * 2);
        // dU = M^T dO + Kt dS' (the 16x16x16 product starts from zero: accumulating it
        // onto a 16x16x32 result still in flight is not covered by the wait states)
        const f32x4 u = dU[c] + mfma16(aT, dob[c], zero4());
        const f32x4 dy = mfma16(tT, pack4(u), zero4());        // dY = Tm^T dU
        nby[c] = pack4(-bt[0] * dy[0], -bt[1] * dy[1], -bt[2] * dy[2], -bt[3] * dy[3]);
      }
      // dS = Diag(Gam) dS' + Qh^T dO - Kh^T Diag(beta) dY
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int s2 = m >> 1, h2 = m & 1;
        const float d1 = st.tot[I][32 * s2 + 8 * p + 4 * h2 + (rr & 3)];
        const int cha = 32 * s2 + 8 * (rr >> 2) + 4 * h2 + (rr & 3);
        const bf16x4 aq = *reinterpret_cast<const bf16x4*>(&st.qrT[cha][16 * I + 4 * p]);
        const bf16x4 ak = *reinterpret_cast<const bf16x4*>(&st.krT[cha][16 * I + 4 * p]);
        const f32x4 dc = {quad_bcast<0>(d1), quad_bcast<1>(d1), quad_bcast<2>(d1),
                          quad_bcast<3>(d1)};
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          f32x4 t_ = D_acc[c][m];
#pragma unroll
          for (int e = 0; e < 4; ++e) t_[e] *= dc[e];
          t_ = mfma16(aq, dob[c], t_);
          D_acc[c][m] = mfma16(ak, nby[c], t_);
        }
      }
    }
    lds_barrier();
  }
  if (b.ds0) {
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ch = 32 * (m >> 1) + 8 * p + 4 * (m & 1) + e;
          b.ds0[state_off + (size_t)ch * DV + col[c]] = D_acc[c][m][e];
        }
  }
}

template <int NS, int NT, bool PER_CHANNEL, bool GDR2>
__global__ __launch_bounds__(64 * (kPrepWaves + NS)) void chunk_bwd_state_kernel(BwdArgs b) {
  constexpr int DV = 16 * NS * NT;
  __shared__ __align__(16) RSmem sm;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rr = lane & 15, p = lane >> 4;
  const ChunkArgs& a = b.f;
  // work item: a chain, or one half of its value columns (the forward's schedule)
  int chain = blockIdx.x, part = 0;
  if (b.plan) {
    if (blockIdx.x >= b.plan[0]) return;
    const uint32_t item = b.plan[1 + blockIdx.x];
    chain = (int)(item >> 2);
    part = (int)(item & 3);
  } else if (NT > 1 && a.split_all) {
    uint32_t c, pt;
    split_item(blockIdx.x, (uint32_t)(a.N * a.H), c, pt);
    chain = (int)c;
    part = (int)pt;
  }
  const int n = chain / a.H, h = chain % a.H;
  const TokenRange tr = token_range(a.cu, n, a.T);
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0;
  const size_t state_off = ((size_t)n * a.H + h) * kDK * DV;
  const size_t hist_off = hist_chain_offset(a, n, h, tr);
  const int nsteps = (tr.len + kC - 1) / kC;
  if (wave < kPrepWaves) {
    const int I = wave;
    const PrepSrc src = prep_src<PER_CHANNEL, GDR2>(a, row0, tr.len, I, lane);
    BlockRegs r;
    if (nsteps > 0) {
      load_block<PER_CHANNEL, GDR2>(r, src, (nsteps - 1) * kC);
      prep_block_rev<GDR2>(sm.st[(nsteps - 1) & 1], sm.qg, sm.kg, r, I, lane);
      wave_lds_fence();
      block_tiles_rev(sm.st[(nsteps - 1) & 1], sm.qg, sm.kg, I, rr, p);
      if (nsteps > 1) load_block<PER_CHANNEL, GDR2>(r, src, (nsteps - 2) * kC);
    }
    lds_barrier();
    for (int s = nsteps - 1; s >= 0; --s) {
      if (s > 0) {
        RStage& st = sm.st[(s - 1) & 1];
        prep_block_rev<GDR2>(st, sm.qg, sm.kg, r, I, lane);
        wave_lds_fence();
        block_tiles_rev(st, sm.qg, sm.kg, I, rr, p);
        if (s > 1) load_block<PER_CHANNEL, GDR2>(r, src, (s - 2) * kC);
      }
      lds_barrier();
    }
  } else {
    __builtin_amdgcn_s_setprio(KDA_STATE_PRIO);
    const int j = wave - kPrepWaves;
    if constexpr (NT > 1) {
      if (part) {  // a half item: NT / 2 tiles per wavefront over one half of the columns
        carry_role<NT / 2, DV>(sm, b, tr, row0, state_off, hist_off, nsteps,
                               (part == 2 ? DV / 2 : 0) + 16 * (NT / 2) * j, lane, rr, p);
        return;
      }
    }
    carry_role<NT, DV>(sm, b, tr, row0, state_off, hist_off, nsteps, 16 * NT * j, lane, rr, p);
  }
}

// ------------------------------------------------------------ launch 3: the gradients

// One workgroup of two wavefronts per pair of 16-token blocks, one wavefront per block.
// The history holds, per pair, the state S_e entering the even block and the gradient dS'_o
// reaching the end of the odd block; the even wavefront reads S_e and the odd one dS'_o, one
// 16-column value tile at a time as stored (lane-native B operands over 32-channel slabs).
// Per tile each first forms, from its own block, the boundary tile the other needs:
//   even: U_e = Tm_e Diag(beta_e) (V_e - Kh_e S_e),  then  S_o = Diag(Gam_e) S_e + Kt_e^T U_e
//   odd:  dY_o = Tm_o^T (M_o^T dO_o + Kt_o dS'_o),
//         then  dS'_e = Diag(Gam_o) dS'_o + Qh_o^T dO_o - Kh_o^T Diag(beta_o) dY_o
// (the forward's state step and the carry across the boundary between the blocks); after
// one barrier each takes the tile it received, finishes its block's columns of Kh S, U, dU
// and dY, and adds the tile's share of every contraction over the value columns (dO S^T,
// Diag(beta) dY S^T, U dS'^T, dO U^T, dY U^T and rowsum(dS' * S)) for all channels, taking
// S and dS' transposed by products with a 0/1 selector (exact in bf16).

template <int DV>
struct GSmem {
  float P[16][kDK];        // decay from the block start through token t; later d log P_t
  float gam[kDK];
  bf16 dor[16][kLDK];      // token rows of dO (dv <= dk columns); later of dq (dk columns)
  bf16 vr[16][kLDK];       // token rows of V (dv columns)
  union {
    struct {               // phases 2-4
      bf16 ut[16][24];     // U, dY, Diag(beta) dY of the current value tile (token rows)
      bf16 yt[16][24];
      bf16 bt[16][24];
      float M[16][17];     // Tril(Qh Kb^T)
      float Tm[16][17];
      float G1[16][17];    // dO U^T
    } w;
    bf16 dkr[16][kLDK];    // phase 4-5: token rows of dk (written after the above are read)
  } u;
  float A[16][17];         // StrictTril(Kh Kb^T)
  float G2[16][17];        // dY U^T
  float beta[16];
  float dlgam[kDK];        // d log Gam
};

// LDS of one pair: each block's scratch; per block, the two channel halves' shares of the
// sums over the channels (the 16 x 16 products of phase 1, and Kh S or Kt dS' of a value
// tile before and after the boundary tiles, by tile parity) and of one decay per head; and
// the boundary tiles, by tile parity and receiver.
struct GHalf {
  union {
    f32x4 mq[2][3][64];     // [half]: Qh Kb^T, Kh Kb^T (column layout), Kh Kb^T (row layout)
    // [parity][half]: Kh S or Kt dS' of the tile, before the boundary tiles and again after
    // them (the second use begins once every wavefront has read the first)
    f32x4 xp[2][2][64];
  };
  float dgh[2][16];         // [half]: the per-token sums of dg (one decay per head)
};
template <int DV>
struct GQuad {
  GSmem<DV> w[2];            // the even block's, the odd block's
  GHalf x[2];
  bf16x8 bnd[2][2][4][64];   // [parity][receiver]: dS'_e for the even, S_o for the odd
};

// Position of work item (pair of 16-token blocks) `slot` of head h: sequence n and pair pr,
// or false when the slot holds no pair. Sequence n's pairs take slots from
// floor(cu[n] / 32) + n on (consecutive sequences never overlap).
__device__ __forceinline__ bool grad_item(const ChunkArgs& a, int slot, int& n, int& pr,
                                          TokenRange& tr) {
  if (!a.cu) {
    const int per = (a.T + 31) / 32;
    n = slot / per;
    pr = slot % per;
    if (n >= a.N) return false;
    tr = token_range(nullptr, n, a.T);
    return true;
  }
  int lo = 0, hi = a.N - 1;  // last sequence whose first slot is <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int first = min(max(a.cu[mid], 0), a.T) / 32 + mid;
    if (first <= slot) lo = mid; else hi = mid - 1;
  }
  n = lo;
  tr = token_range(a.cu, n, a.T);
  pr = slot - (tr.t0 / 32 + n);
  return pr >= 0 && pr * 32 < tr.len;
}

// Selector of channels 16 hh + n out of a 32-channel slab, as the B operand of a
// 16x16x32 product: with an S tile as the A operand (lane 16 p + r holds channels
// 8 p + i of column r) the product is the tile transposed, D[4p + e][n] = S[16 hh + n]
// [column 4 p + e], exactly (one nonzero term per entry).
__device__ __forceinline__ bf16x8 selector(int hh, int rr, int p) {
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = static_cast<bf16>(8 * p + i == 16 * hh + rr ? 1.f : 0.f);
  return b;
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float (&x)[8]) {
  return cat8(pack4(x[0], x[1], x[2], x[3]), pack4(x[4], x[5], x[6], x[7]));
}

// Selector of the channels 8 (n / 4) + 4 hh + n % 4 (n < 16) of a 32-channel slab: with
// token rows of an operand X as the A operand of a 16x16x32 product (lane 16 p + r holds
// channels 8 p + i of token r), D[4p + e][n] = X[token 4p + e][that channel], which is, in
// lane order, the A operand of X^T's channel tile 2 ks + hh for a 16x16x16 product.
__device__ __forceinline__ bf16x8 tile_selector(int hh, int rr, int p) {
  const int c = 8 * (rr >> 2) + 4 * hh + (rr & 3);
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = static_cast<bf16>(8 * p + i == c ? 1.f : 0.f);
  return b;
}

// GDR2: the Gated Delta Rule-2 gates. The read-side key Kh is then (b * k) P, beta is 1,
// R = w * V - Kh S, dV = w * dY, and the gradients of the gates are d erase = k P * dKh and
// d write = V * dY (instead of dbeta).
// Four wavefronts per workgroup: the pair's even and odd block (odd = wave / 2), each split
// over two halves of the key channels (hc = wave % 2: slabs 2 hc and 2 hc + 1, channel tiles
// 4 hc .. 4 hc + 3, channels 64 hc .. 64 hc + 63). A half holds its slabs of the stored tile,
// the row operands and the contraction sums; contractions over the channels (Kh S, Kt dS'
// and the 16 x 16 products of the row operands) are summed over the two halves through LDS,
// and the 16 x 16 steps that follow them (U, dY, the block inverse) run in both halves.
// About 76 KB of LDS: two workgroups, two wavefronts per SIMD, at most 256 registers each.
template <int DV, bool PER_CHANNEL, bool GDR2>
__global__ __attribute__((amdgpu_waves_per_eu(2))) __launch_bounds__(256) void
chunk_bwd_grad_kernel(BwdArgs b, int slots) {
  constexpr int NCT = DV / 16;   // value tiles of the block
  __shared__ __align__(16) GQuad<DV> sp;
  const ChunkArgs& a = b.f;
  // the wavefront's block within the pair and channel half, uniform across the wavefront
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int odd = wave >> 1, hc = wave & 1;
  const int lane = threadIdx.x & 63;
  const int rr = lane & 15, p = lane >> 4;
  GSmem<DV>& sm = sp.w[odd];
  GHalf& xs = sp.x[odd];
  const int h = blockIdx.x / slots, slot = blockIdx.x % slots;
  int n, pr;
  TokenRange tr;
  if (!grad_item(a, slot, n, pr, tr)) return;   // all four wavefronts leave together
  const int blk = 2 * pr + odd;
  // tokens of this block in the sequence: 0 for the odd block of a sequence's last pair when
  // its block count is odd; every view of that block is then empty (zeros), which makes it
  // the identity block, and the stored gradient is the one reaching the even block's end
  // (made a scalar explicitly: the clamp is a vector instruction, and a vector operand in
  // the buffer descriptors below would put each of their loads in a loop over lanes)
  const int len = __builtin_amdgcn_readfirstlane(max(0, min(16, tr.len - 16 * blk)));
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0 + 16 * (size_t)blk;
  const size_t hoff = hist_chain_offset(a, n, h, tr) + (size_t)pr * kDK * DV * 2;
  const rsrc_t qs = make_rsrc(static_cast<const bf16*>(a.q) + row0 * kDK, len * kDK * 2);
  const rsrc_t ks_ = make_rsrc(static_cast<const bf16*>(a.k) + row0 * kDK, len * kDK * 2);
  const rsrc_t vs = make_rsrc(static_cast<const bf16*>(a.v) + row0 * DV, len * DV * 2);
  // the stored matrix of this block: S_e (even) or dS'_o (odd)
  const rsrc_t hm = make_rsrc(static_cast<const char*>(odd ? b.hist_ds : b.hist_s) + hoff,
                              kDK * DV * 2);
  const rsrc_t es = make_rsrc(a.erase + (GDR2 ? row0 * kDK : 0), GDR2 ? len * kDK * 4 : 0);
  const rsrc_t ws_ = make_rsrc(a.write + (GDR2 ? row0 * DV : 0), GDR2 ? len * DV * 4 : 0);

  // this half's slabs of the stored matrix's value tiles 0 and 1 (prefetched two tiles
  // ahead in the loop below)
  bf16x8 hb[2], hn[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ks = 2 * hc + j;
    hb[j] = __builtin_bit_cast(bf16x8, ld_b128(hm, (uint32_t)((ks * 64 + lane) * 16)));
    hn[j] = __builtin_bit_cast(bf16x8, ld_b128(hm, (uint32_t)(((4 + ks) * 64 + lane) * 16)));
  }
  // q and k of token rr, channels 32 ks + 8 p + i of this half's slabs: the row operands
  // (kept for the per-channel step after the tiles)
  bf16x8 q8[2], k8[2];
  f32x4 e8[2][2];   // erase gates of the same elements (Gated Delta Rule-2)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t off = (uint32_t)(rr * kDK + 32 * (2 * hc + j) + 8 * p);
    q8[j] = __builtin_bit_cast(bf16x8, ld_b128(qs, off * 2));
    k8[j] = __builtin_bit_cast(bf16x8, ld_b128(ks_, off * 2));
    if (GDR2) {
      e8[j][0] = ld_b128(es, off * 4);
      e8[j][1] = ld_b128(es, off * 4 + 16);
    }
  }

  // ---- 0. decay of this half's channels (one per lane), half of the dO and V rows, beta.
  // Every load is issued before the first use: bounded reads past the block's last token
  // return g = 0.
  {
    const rsrc_t ds = make_rsrc(static_cast<const bf16*>(b.dout) + row0 * DV, len * DV * 2);
    const rsrc_t gs = make_rsrc(a.g + row0 * (PER_CHANNEL ? kDK : 1),
                                len * (PER_CHANNEL ? kDK : 1) * 4);
    constexpr int NV = 16 * DV / 8 / 128;   // 16-byte row pieces per lane (half the rows)
    f32x4 dov[NV], vov[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = lane + 64 * (2 * j + hc), tt = i / (DV / 8), cc = 8 * (i % (DV / 8));
      dov[j] = ld_b128(ds, (uint32_t)(tt * DV + cc) * 2);
      vov[j] = ld_b128(vs, (uint32_t)(tt * DV + cc) * 2);
    }
    const float bv = GDR2 ? 1.f : ld_b32(make_rsrc(a.beta + row0, len * 4), (lane & 15) * 4);
    float gv[16];
    const int c = 64 * hc + lane;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      gv[t] = ld_b32(gs, (uint32_t)(PER_CHANNEL ? t * kDK + c : t) * 4);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = lane + 64 * (2 * j + hc), tt = i / (DV / 8), cc = 8 * (i % (DV / 8));
      *reinterpret_cast<f32x4*>(&sm.dor[tt][cc]) = dov[j];
      *reinterpret_cast<f32x4*>(&sm.vr[tt][cc]) = vov[j];
    }
    float run = 1.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      run *= __expf(gv[t]);
      sm.P[t][c] = run;
    }
    sm.gam[c] = run;
    if (hc == 0 && lane < 16) sm.beta[lane] = bv;
  }
  wave_lds_fence();

  // ---- 1. row operands of token rr (bf16) on this half's slabs: Qh, Kh (the read-side
  // key), Kb = k / P, Kt; this half's share of the 16 x 16 products over the channels; the
  // transposed operands of this half's channel tiles for the boundary tile (Kt_e^T in the
  // even block, Qh_o^T and Kh_o^T in the odd one)
  bf16x8 ah[2], at[2];
  bf16x4 tr1[4], tr2[4];
  {
    f32x4 accq = zero4(), acck = zero4(), acct = zero4();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c0 = 32 * (2 * hc + j) + 8 * p;
      float qh[8], kh[8], kb[8], kt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float P = sm.P[rr][c0 + i], G = sm.gam[c0 + i];
        const float rp = __builtin_amdgcn_rcpf(P);
        const float kf = static_cast<float>(k8[j][i]);
        qh[i] = static_cast<float>(q8[j][i]) * P;
        kh[i] = kf * P * (GDR2 ? e8[j][i >> 2][i & 3] : 1.f);
        kb[i] = kf * rp;
        kt[i] = kb[i] * G;
      }
      const bf16x8 bq = to_bf16x8(qh), bc = to_bf16x8(kb);
      ah[j] = to_bf16x8(kh);
      at[j] = to_bf16x8(kt);
      accq = mfma32(bq, bc, accq);        // (Qh Kb^T)[4p + e][rr], this half's channels
      acck = mfma32(ah[j], bc, acck);     // (Kh Kb^T)[4p + e][rr]
      acct = mfma32(bc, ah[j], acct);     // (Kh Kb^T)[rr][4p + e]
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8 ts = tile_selector(hh, rr, p);
        if (odd) {
          tr1[2 * j + hh] = pack4(mfma32(bq, ts, zero4()));
          tr2[2 * j + hh] = pack4(mfma32(ah[j], ts, zero4()));
        } else {
          tr1[2 * j + hh] = pack4(mfma32(at[j], ts, zero4()));
          tr2[2 * j + hh] = bf16x4{};
        }
      }
    }
    xs.mq[hc][0][lane] = accq;
    xs.mq[hc][1][lane] = acck;
    xs.mq[hc][2][lane] = acct;
  }
  lds_barrier();   // both halves' shares, the dO and V rows and beta are written
  // ---- 2. M, A and Tm of the block (in both halves; both write the same values)
  {
    f32x4 accq, acck, acct;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      accq[e] = xs.mq[0][0][lane][e] + xs.mq[1][0][lane][e];
      acck[e] = xs.mq[0][1][lane][e] + xs.mq[1][1][lane][e];
      acct[e] = xs.mq[0][2][lane][e] + xs.mq[1][2][lane][e];
    }
    f32x4 nc, nr;
    const float brr = sm.beta[rr];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * p + e;
      sm.u.w.M[i][rr] = rr <= i ? accq[e] : 0.f;
      sm.A[i][rr] = rr < i ? acck[e] : 0.f;
      nc[e] = rr < i ? sm.beta[i] * acck[e] : 0.f;
      nr[e] = i < rr ? brr * acct[e] : 0.f;
    }
    const f32x4 inv = unit_lower_inverse(nc, nr, rr, p);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.u.w.Tm[4 * p + e][rr] = inv[e];
  }
  lds_barrier();   // every half has read the shares (their storage holds the tiles' sums next)

  // ---- 3. the value tiles
  f32x4 C1[4], C2[4], C3[4], g1 = zero4(), g2 = zero4();
  float r2[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    C1[m] = C2[m] = C3[m] = zero4();
    r2[m] = 0.f;
  }
  f32x4 r1 = zero4();
  const rsrc_t vd = make_rsrc(static_cast<bf16*>(b.dv) + row0 * DV, len * DV * 2);
  // the write gates of value tile ct in the accumulator layout (token 4p + e), loaded one
  // tile ahead (Gated Delta Rule-2)
  f32x4 wnext;
  auto load_write_gates = [&](int ct) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wnext[e] = GDR2 ? ld_b32(ws_, (uint32_t)((4 * p + e) * DV + 16 * ct + rr) * 4) : 1.f;
  };
  load_write_gates(0);
  // Gated Delta Rule-2: the erase gates of token 4 p + e, channel 16 (4 hc + m) + rr for the
  // per-channel step after the tiles (loaded now, so that the tiles cover their latency)
  float e4[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      e4[m][e] = GDR2 ? ld_b32(es, (uint32_t)((4 * p + e) * kDK + 16 * (4 * hc + m) + rr) * 4)
                      : 1.f;
  // the tile loop, compiled separately for each block of the pair (one loop per wavefront,
  // no branch on the block inside it)
  auto tiles = [&](auto role) {
    constexpr int ODD = decltype(role)::value;
    // the block's operands that every tile uses, held in registers across the tiles: Tm,
    // Tm^T, M^T, beta, the transposes' selectors and the decay Gam of this half's state tile
    // rows (channel tile 2 j + hh: 32 (2 hc + j) + 8 p + 4 hh + e)
    bf16x4 tA, tT, mT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tA[i] = static_cast<bf16>(sm.u.w.Tm[rr][4 * p + i]);   // Tm row rr
      tT[i] = static_cast<bf16>(sm.u.w.Tm[4 * p + i][rr]);   // Tm^T row rr
      mT[i] = static_cast<bf16>(sm.u.w.M[4 * p + i][rr]);    // M^T row rr
    }
    const f32x4 btv = *reinterpret_cast<const f32x4*>(&sm.beta[4 * p]);
    const bf16x8 sel[2] = {selector(0, rr, p), selector(1, rr, p)};
    f32x4 gmr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      gmr[m] = *reinterpret_cast<const f32x4*>(
          &sm.gam[32 * (2 * hc + (m >> 1)) + 8 * p + 4 * (m & 1)]);
#pragma unroll 1
    for (int ct = 0; ct < NCT; ++ct) {
      const int col = 16 * ct + rr, par = ct & 1;
      // V and the write gates of this tile (token 4p + e, column col)
      f32x4 vcol, wcol;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vcol[e] = static_cast<float>(sm.vr[4 * p + e][col]);
        wcol[e] = GDR2 ? wnext[e] : 1.f;
      }
      if (GDR2 && ct + 1 < NCT) load_write_gates(ct + 1);
      bf16x4 dob;
#pragma unroll
      for (int e = 0; e < 4; ++e) dob[e] = sm.dor[4 * p + e][col];
      // this half's slabs of the block's S and dS' of the tile (sc, dc)
      bf16x8 sc[2], dc[2];
      f32x4 R, U, dY;
      // A: this half's share of Kh S_e (even) or Kt dS'_o (odd), from the stored slabs
      {
        f32x4 part = zero4();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (!ODD) {
            sc[j] = hb[j];
            part = mfma32(ah[j], sc[j], part);
          } else {
            dc[j] = hb[j];
            part = mfma32(at[j], dc[j], part);
          }
        }
        xs.xp[par][hc][lane] = part;
      }
      // the stored slabs two tiles ahead (past the last tile the loads read zeros)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        hb[j] = hn[j];
        hn[j] = __builtin_bit_cast(
            bf16x8, ld_b128(hm, (uint32_t)((((ct + 2) * 4 + 2 * hc + j) * 64 + lane) * 16)));
      }
      lds_barrier();   // both halves' shares are written
      f32x4 whole;
#pragma unroll
      for (int e = 0; e < 4; ++e) whole[e] = xs.xp[par][0][lane][e] + xs.xp[par][1][lane][e];
      if constexpr (!ODD) {   // U_e, then this half's rows of the odd block's entering state
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          R[e] = wcol[e] * vcol[e] - whole[e];
          x[e] = btv[e] * R[e];
        }
        U = mfma16(tA, pack4(x), zero4());
        const bf16x4 ub = pack4(U);
#pragma unroll
        for (int j = 0; j < 2; ++j) {   // S_o = Diag(Gam_e) S_e + Kt_e^T U_e
          f32x4 acc[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const f32x4 gm = gmr[2 * j + hh];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[hh][e] = gm[e] * static_cast<float>(sc[j][4 * hh + e]);
            acc[hh] = mfma16(tr1[2 * j + hh], ub, acc[hh]);
          }
          sp.bnd[par][1][2 * hc + j][lane] = cat8(pack4(acc[0]), pack4(acc[1]));
        }
      } else {      // dY_o, then this half's rows of the even block's leaving gradient
        const f32x4 dU = whole + mfma16(mT, dob, zero4());
        dY = mfma16(tT, pack4(dU), zero4());
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = -btv[e] * dY[e];
        const bf16x4 yb = pack4(y);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // dS'_e = Diag(Gam_o) dS'_o + Qh_o^T dO_o - Kh_o^T Diag(beta_o) dY_o
          f32x4 acc[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const f32x4 gm = gmr[2 * j + hh];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[hh][e] = gm[e] * static_cast<float>(dc[j][4 * hh + e]);
            acc[hh] = mfma16(tr1[2 * j + hh], dob, acc[hh]);
            acc[hh] = mfma16(tr2[2 * j + hh], yb, acc[hh]);
          }
          sp.bnd[par][0][2 * hc + j][lane] = cat8(pack4(acc[0]), pack4(acc[1]));
        }
      }
      lds_barrier();   // the boundary tiles of this value tile are written
      // B: this half's share of Kt dS'_e (even) or Kh S_o (odd), from the received slabs
      {
        f32x4 part = zero4();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (!ODD) {
            dc[j] = sp.bnd[par][0][2 * hc + j][lane];
            part = mfma32(at[j], dc[j], part);
          } else {
            sc[j] = sp.bnd[par][1][2 * hc + j][lane];
            part = mfma32(ah[j], sc[j], part);
          }
        }
        xs.xp[par][hc][lane] = part;
      }
      lds_barrier();   // both halves' shares are written
#pragma unroll
      for (int e = 0; e < 4; ++e) whole[e] = xs.xp[par][0][lane][e] + xs.xp[par][1][lane][e];
      if constexpr (!ODD) {   // dY_e
        const f32x4 dU = whole + mfma16(mT, dob, zero4());
        dY = mfma16(tT, pack4(dU), zero4());
      } else {      // U_o
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          R[e] = wcol[e] * vcol[e] - whole[e];
          x[e] = btv[e] * R[e];
        }
        U = mfma16(tA, pack4(x), zero4());
      }
      // the tile rows of U, dY and Diag(beta) dY (both halves write the same values, each
      // then reads back what it wrote)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.u.w.ut[4 * p + e][rr] = static_cast<bf16>(U[e]);
        sm.u.w.yt[4 * p + e][rr] = static_cast<bf16>(dY[e]);
        sm.u.w.bt[4 * p + e][rr] = static_cast<bf16>((GDR2 ? wcol[e] : btv[e]) * dY[e]);
        r1[e] += dY[e] * R[e];
        if (GDR2 && hc == 0 && 4 * p + e < len)   // d write = V * dY
          b.dwrite[(row0 + 4 * p + e) * DV + col] = vcol[e] * dY[e];
      }
      wave_lds_fence();
      // dV = Diag(beta) dY (w * dY): this tile's 16 token rows of 16 columns
      if (hc == 0 && lane < 32) {
        const int t = lane >> 1, c8 = 8 * (lane & 1);
        st_b128(vd, (uint32_t)(t * DV + 16 * ct + c8) * 2,
                *reinterpret_cast<const bf16x8*>(&sm.u.w.bt[t][c8]));
      }
      // the tile's share of the contractions over the value columns (k = column
      // 16 ct + 4p + i), for this half's channel tiles
      const bf16x4 ao = *reinterpret_cast<const bf16x4*>(&sm.dor[rr][16 * ct + 4 * p]);
      // beta = 1 with the Gated Delta Rule-2 gates: Diag(beta) dY is dY itself
      const bf16x4 ay =
          *reinterpret_cast<const bf16x4*>(GDR2 ? &sm.u.w.yt[rr][4 * p] : &sm.u.w.bt[rr][4 * p]);
      const bf16x4 au = *reinterpret_cast<const bf16x4*>(&sm.u.w.ut[rr][4 * p]);
      const bf16x4 ayy = *reinterpret_cast<const bf16x4*>(&sm.u.w.yt[rr][4 * p]);
      g1 = mfma16(ao, au, g1);     // (dO U^T)[4p + e][rr] (used from half 0)
      g2 = mfma16(ayy, au, g2);    // (dY U^T)[4p + e][rr]
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int m = 2 * j + hh;   // channel tile 4 hc + m: channels 16 (4 hc + m) + n
          const f32x4 st = mfma32(sc[j], sel[hh], zero4());   // S[16 (4 hc + m) + rr][16 ct + 4p + e]
          const f32x4 dt = mfma32(dc[j], sel[hh], zero4());
          const bf16x4 sb4 = pack4(st), db4 = pack4(dt);
          C1[m] = mfma16(ao, sb4, C1[m]);   // (dO S^T)[4p + e][16 (4 hc + m) + rr]
          C2[m] = mfma16(ay, sb4, C2[m]);   // (Diag(beta) dY S^T)
          C3[m] = mfma16(au, db4, C3[m]);   // (U dS'^T)
#pragma unroll
          for (int e = 0; e < 4; ++e) r2[m] += st[e] * dt[e];
        }
    }
  };
  if (odd) tiles(std::integral_constant<int, 1>{});
  else tiles(std::integral_constant<int, 0>{});
  // reductions: r1 over the 16 columns of each lane group, r2 over the lane groups
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = r1[e];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    r1[e] = v;   // lane 16 p + r: token 4 p + e
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    r2[m] += __shfl_xor(r2[m], 16, 64);
    r2[m] += __shfl_xor(r2[m], 32, 64);
  }
  lds_barrier();   // both halves are done with the last tile's rows (G1 shares their storage)
  if (hc == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.u.w.G1[4 * p + e][rr] = g1[e];
      sm.G2[4 * p + e][rr] = g2[e];
    }
  }
  lds_barrier();   // G1 and G2 are written

  // ---- 4. the 16 x 16 corrections and the chain rule through the decay, per channel tile
  bf16x4 dmr, dar, dmT, daT;   // dM, dA rows rr and columns rr
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s_ = 4 * p + i;
    dmr[i] = static_cast<bf16>(s_ <= rr ? sm.u.w.G1[rr][s_] : 0.f);
    dar[i] = static_cast<bf16>(s_ < rr ? -sm.beta[rr] * sm.G2[rr][s_] : 0.f);
    dmT[i] = static_cast<bf16>(rr <= s_ ? sm.u.w.G1[s_][rr] : 0.f);
    daT[i] = static_cast<bf16>(rr < s_ ? -sm.beta[s_] * sm.G2[s_][rr] : 0.f);
  }
  lds_barrier();   // G1 is read by both halves before dk overwrites it (same storage)
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int ch = 16 * (4 * hc + m) + rr;
    const float G = sm.gam[ch];
    // q and k of token 4 p + e, channel ch: the rows transposed by the selector (exact)
    const bf16x8 sel = selector(m & 1, rr, p);
    const f32x4 qT = mfma32(q8[m >> 1], sel, zero4());
    const f32x4 kT = mfma32(k8[m >> 1], sel, zero4());
    float P[4], qf[4], kf[4], bf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      P[e] = sm.P[4 * p + e][ch];
      qf[e] = qT[e];
      kf[e] = kT[e];
      bf[e] = e4[m][e];
    }
    // operands with k = token (4p + i) and n = this channel
    bf16x4 bkb, bkh, bqh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float rp = __builtin_amdgcn_rcpf(P[i]);
      bkb[i] = static_cast<bf16>(kf[i] * rp);
      bkh[i] = static_cast<bf16>(kf[i] * P[i] * bf[i]);
      bqh[i] = static_cast<bf16>(qf[i] * P[i]);
    }
    const f32x4 dQh = C1[m] + mfma16(dmr, bkb, zero4());
    const f32x4 dKh = mfma16(dar, bkb, zero4()) - C2[m];
    const f32x4 dKb = mfma16(daT, bkh, zero4()) + mfma16(dmT, bqh, zero4());
    const f32x4 dKt = C3[m];
    float lg = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * p + e;
      const float rp = __builtin_amdgcn_rcpf(P[e]);
      const float qh = qf[e] * P[e], kh = kf[e] * P[e] * bf[e], kb = kf[e] * rp, kt = kb * G;
      sm.dor[t][ch] = static_cast<bf16>(dQh[e] * P[e]);                                 // dq
      sm.u.dkr[t][ch] = static_cast<bf16>(dKh[e] * P[e] * bf[e] + (dKb[e] + dKt[e] * G) * rp);
      sm.P[t][ch] = dQh[e] * qh + dKh[e] * kh - dKb[e] * kb - dKt[e] * kt;             // d log P
      if (GDR2 && t < len) b.derase[(row0 + t) * kDK + ch] = dKh[e] * kf[e] * P[e];  // d erase
      lg += dKt[e] * kt;
    }
    lg += __shfl_xor(lg, 16, 64);
    lg += __shfl_xor(lg, 32, 64);
    if (p == 0) sm.dlgam[ch] = lg + G * r2[m];
  }
  wave_lds_fence();

  // ---- 5. outputs: this half's channels of the dq, dk rows; dg (suffix sums); dbeta
  {
    const rsrc_t qd = make_rsrc(static_cast<bf16*>(b.dq) + row0 * kDK, len * kDK * 2);
    const rsrc_t kd = make_rsrc(static_cast<bf16*>(b.dk) + row0 * kDK, len * kDK * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = lane + 64 * i;   // 128 pieces of 8 channels (16 tokens x 8 pieces)
      const int t = idx >> 3, c8 = 64 * hc + 8 * (idx & 7);
      const uint32_t off = (uint32_t)(t * kDK + c8) * 2;
      st_b128(qd, off, *reinterpret_cast<const bf16x8*>(&sm.dor[t][c8]));
      st_b128(kd, off, *reinterpret_cast<const bf16x8*>(&sm.u.dkr[t][c8]));
    }
  }
  float dgs[16];   // the suffix sums of this lane's channel 64 hc + lane
  {
    const int c = 64 * hc + lane;
    float acc = sm.dlgam[c];
#pragma unroll
    for (int t = 15; t >= 0; --t) {
      acc += sm.P[t][c];
      dgs[t] = acc;
      if (PER_CHANNEL && t < len) b.dg[(row0 + t) * kDK + c] = acc;
    }
  }
  if (!PER_CHANNEL) {   // one decay per head: the sum over the channels of both halves
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float v = dgs[t];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      dgs[t] = v;
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < 16; ++t) xs.dgh[hc][t] = dgs[t];
    }
  }
  lds_barrier();   // (one decay per head) both halves' sums are written
  if (!PER_CHANNEL && hc == 0 && lane < 16 && lane < len)
    b.dg[row0 + lane] = xs.dgh[0][lane] + xs.dgh[1][lane];
  if (!GDR2 && hc == 0) {
    // dbeta_t = sum_j dY_tj R_tj - sum_s A_ts (dY U^T)_ts; lane 16 p holds token 4 p + e
    if (rr == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * p + e;
        float acc = r1[e];
        for (int s_ = 0; s_ < t; ++s_) acc -= sm.A[t][s_] * sm.G2[t][s_];
        if (t < len) b.dbeta[row0 + t] = acc;
      }
    }
  }
}

}  // namespace

// Row copies for the dk = 64 backward, which runs the dk = 128 kernels on key-side arrays
// padded with zero channels: destination row r takes the first min(w_src, w_dst) elements of
// source row r, then zeros up to w_dst (the elements are moved as raw bits; zero bits are a
// zero of either element type).
template <typename E>
__global__ void pad_rows_kernel(const E* __restrict__ src, E* __restrict__ dst, long long rows,
                                int w_src, int w_dst) {
  const long long n = rows * w_dst;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const long long r = i / w_dst;
    const int c = (int)(i - r * w_dst);
    dst[i] = c < w_src ? src[r * w_src + c] : E(0);
  }
}

hipError_t launch_pad_rows(const void* src, void* dst, long long rows, int w_src, int w_dst,
                           int elem_bytes, hipStream_t stream) {
  if (rows <= 0 || w_dst <= 0) return hipSuccess;
  const long long n = rows * w_dst;
  const unsigned blocks = (unsigned)std::min<long long>((n + 255) / 256, 1 << 16);
  if (elem_bytes == 2)
    pad_rows_kernel<uint16_t><<<blocks, 256, 0, stream>>>(static_cast<const uint16_t*>(src),
                                                         static_cast<uint16_t*>(dst), rows,
                                                         w_src, w_dst);
  else
    pad_rows_kernel<uint32_t><<<blocks, 256, 0, stream>>>(static_cast<const uint32_t*>(src),
                                                         static_cast<uint32_t*>(dst), rows,
                                                         w_src, w_dst);
  return hipGetLastError();
}

bool chunk_bwd_supports(int dk, int dv, int T) {
  // the forward's bounds, and one chain's state history addressable by a buffer descriptor
  return chunk_mfma_supports(dk, dv, T) && ((long long)T + 64) * 8 * dv < (1ll << 31);
}

size_t chunk_bwd_hist_bytes(int N, int H, int T, int dv, bool packed) {
  const size_t tokens = packed ? (size_t)T + 64 * (size_t)N : (size_t)N * (((size_t)T + 63) / 64 * 64);
  return (size_t)H * tokens * (kDK / 16) * (size_t)dv;  // hist_chain_offset's layout
}

namespace {

template <bool GDR2>
hipError_t launch_carry(BwdArgs& b, bool per_channel, unsigned chains, hipStream_t stream) {
  const ChunkArgs& a = b.f;
  const unsigned threads = 64 * (kPrepWaves + 4);
  if (a.dv == 128) {
    if (per_channel) chunk_bwd_state_kernel<4, 2, true, GDR2><<<chains, threads, 0, stream>>>(b);
    else chunk_bwd_state_kernel<4, 2, false, GDR2><<<chains, threads, 0, stream>>>(b);
  } else {
    if (per_channel) chunk_bwd_state_kernel<4, 1, true, GDR2><<<chains, threads, 0, stream>>>(b);
    else chunk_bwd_state_kernel<4, 1, false, GDR2><<<chains, threads, 0, stream>>>(b);
  }
  return hipGetLastError();
}

template <bool GDR2>
hipError_t launch_grad(BwdArgs& b, bool per_channel, int slots, hipStream_t stream) {
  const ChunkArgs& a = b.f;
  const unsigned grid = (unsigned)slots * a.H;
  if (a.dv == 128) {
    if (per_channel) chunk_bwd_grad_kernel<128, true, GDR2><<<grid, 256, 0, stream>>>(b, slots);
    else chunk_bwd_grad_kernel<128, false, GDR2><<<grid, 256, 0, stream>>>(b, slots);
  } else {
    if (per_channel) chunk_bwd_grad_kernel<64, true, GDR2><<<grid, 256, 0, stream>>>(b, slots);
    else chunk_bwd_grad_kernel<64, false, GDR2><<<grid, 256, 0, stream>>>(b, slots);
  }
  return hipGetLastError();
}

// A second stream per device (default priority, created once) for the state history, which
// runs at the same time as the reverse carry: the carry does not read the states.
hipStream_t side_stream() {
  static std::mutex mu;
  static hipStream_t cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev] && hipStreamCreateWithFlags(&cache[dev], hipStreamNonBlocking) != hipSuccess)
    cache[dev] = nullptr;
  return cache[dev];
}

}  // namespace

hipError_t launch_chunk_bwd(const BwdArgs& args, bool per_channel, hipStream_t stream) {
  BwdArgs b = args;
  ChunkArgs& a = b.f;
  if (!chunk_bwd_supports(a.dk, a.dv, a.T)) return hipErrorInvalidValue;
  a.sT = nullptr;
  a.plan = a.cu ? b.plan : nullptr;
  b.plan = a.plan;
  // the work list of packed sequences, shared by the history and the carry
  hipError_t e = launch_chunk_plan(a, stream);
  if (e != hipSuccess) return e;
  const bool can_split = a.dv == 128;
  unsigned chains = (unsigned)a.N * a.H;
  a.split_all = 0;
  if (!b.plan && can_split && a.cus > 0 && 2ll * a.N * a.H <= a.cus) {
    a.split_all = 1;
    chains *= 2;
  }
  // one workgroup per pair of 16-token blocks (grad_item)
  const int slots = a.cu ? a.T / 32 + a.N + 1 : a.N * ((a.T + 31) / 32);
  // 1. the states entering every pair of blocks, on the side stream, and 2. the carry,
  // recording dS' at the end of every pair; then 3. the gradients of every block, after both
  ChunkArgs h = b.f;
  h.hist = b.hist_s;
  h.split_all = 0;  // the history launch decides its own split
  // The fork and join events belong to this call (two calls enqueued from different host
  // threads must not re-record each other's events); the guard destroys them on every path.
  // Destroying an event that a stream still waits on is allowed: the wait keeps its target.
  struct EventPair {
    hipEvent_t forked = nullptr, joined = nullptr;
    ~EventPair() {
      if (forked) (void)hipEventDestroy(forked);
      if (joined) (void)hipEventDestroy(joined);
    }
  } ev;
  hipStream_t side = side_stream();
  if (side && (hipEventCreateWithFlags(&ev.forked, hipEventDisableTiming) != hipSuccess ||
               hipEventCreateWithFlags(&ev.joined, hipEventDisableTiming) != hipSuccess))
    side = nullptr;  // no events: run the history on the caller's stream instead
  if (side) {
    if ((e = hipEventRecord(ev.forked, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(side, ev.forked, 0)) != hipSuccess) return e;
  }
  e = launch_chunk_mfma_hist(h, per_channel, side ? side : stream, false);
  if (e == hipSuccess)
    e = a.erase ? launch_carry<true>(b, per_channel, chains, stream)
                : launch_carry<false>(b, per_channel, chains, stream);
  if (side) {
    // join even after a failed launch, so that the caller's stream never runs ahead of
    // work already enqueued on the side stream
    hipError_t e2 = hipEventRecord(ev.joined, side);
    if (e2 == hipSuccess) e2 = hipStreamWaitEvent(stream, ev.joined, 0);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return e;
  return a.erase ? launch_grad<true>(b, per_channel, slots, stream)
                 : launch_grad<false>(b, per_channel, slots, stream);
}

}  // namespace kda
