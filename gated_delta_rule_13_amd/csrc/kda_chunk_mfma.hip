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
//
// Below the kernel: the work list of packed sequences (chunk_plan_kernel), the segment plan
// that cuts long sequences (chunk_segplan_kernel, seg_chain_kernel, seg_correct_kernel), the
// two-pass segmented scan of dv = 64 (seg_combine_kernel), and the host launchers.
#include <stddef.h>

#include <algorithm>

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
constexpr int kModeTransOut = 5;  // see state_role
constexpr int kModePair = 4;  // launch of both kModeState and kModeTrans items (see the kernel)
constexpr int kModeSeg = 6;   // launch of a segment plan (see chunk_segplan_kernel)
// Segment plan (chunk_segplan_kernel) in the workspace, as 32-bit words: a header of kSegHdr
// words ([0] items, [1] segment length X in 64-token chunks or 0 without segments, [2]
// segments over all sequences, [3] correction units per head, [4] rows of carried-back
// queries per head), then segbase[N + 1] (the first segment of sequence n: its segments are
// slots segbase[n] .. segbase[n + 1] - 1), corr_off[cap + 1] (the first correction unit of
// slot s), qoff[cap + 1] (the first carried-back-query row of slot s) and two words per
// item: ((n * H + h) << 2) | part, and (segment << 2) | kind. cap is the slot capacity the
// workspace was laid out for (ChunkArgs::seg_slots).
constexpr int kSegWhole = 0, kSegFirst = 1, kSegZero = 2, kSegTrans = 3;  // item kinds
constexpr int kSegHdr = 8;
__host__ __device__ inline size_t segplan_corr_off(int N) { return kSegHdr + (size_t)N + 1; }
__host__ __device__ inline size_t segplan_qoff_off(int N, int cap) {
  return segplan_corr_off(N) + (size_t)cap + 1;
}
__host__ __device__ inline size_t segplan_items_off(int N, int cap) {
  return segplan_qoff_off(N, cap) + (size_t)cap + 1;
}

// Issue priority (s_setprio) of the state wavefronts relative to the prep wavefronts
// (priority 0) on the same SIMD, by gate kind, as measured on the packed T = 65536 workloads:
// with one decay per key channel and the beta gate (KDA) equal priority was up to 3% faster
// than priority 1, 2 or 3 and never slower; with the Gated Delta Rule-2 gates or one decay
// per head, priority 3 was 3-7% faster than equal priority.
#ifndef KDA_STATE_PRIO
#define KDA_STATE_PRIO 3
#endif
#ifndef KDA_STATE_PRIO_KDA
#define KDA_STATE_PRIO_KDA 0
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
// Without NEEDQ (a pass that writes no outputs) the query operand is not formed.
template <bool GDR2, bool NEEDQ = true>
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
      qr[j] = NEEDQ ? static_cast<float>(r.q[u][j]) * run[j] : 0.f;
      kr[j] = static_cast<float>(r.k[u][j]) * (GDR2 ? r.b[u][j] * run[j] : run[j]);
    }
    if (NEEDQ) *reinterpret_cast<bf16x4*>(&st.qr[t][4 * cq]) = pack4(qr);
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
// strictly lower (unit_lower_inverse); A_qk only when NEEDQ.
template <bool NEEDQ = true>
__device__ __forceinline__ void block_tiles(Stage& st, const bf16 (*kd)[kLDK], int I, int rr,
                                            int p) {
  bf16x8 bq[4], bk[4], bc[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = 32 * ks + 8 * p;
    if (NEEDQ) bq[ks] = *reinterpret_cast<const bf16x8*>(&st.qr[16 * I + rr][ch]);
    bk[ks] = *reinterpret_cast<const bf16x8*>(&st.kr[16 * I + rr][ch]);
    bc[ks] = *reinterpret_cast<const bf16x8*>(&kd[16 * I + rr][ch]);
  }
  f32x4 accq = zero4(), acck = zero4(), acct = zero4();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (NEEDQ) accq = mfma32(bq[ks], bc[ks], accq);   // A_qk[i][j], lane holds i = 4p + e, j = rr
    acck = mfma32(bk[ks], bc[ks], acck);   // A_kk[i][j]
    acct = mfma32(bc[ks], bk[ks], acct);   // A_kk[j][i]: lane holds A_kk[rr][4p + e]
  }
  f32x4 nc, nr;
  const float brr = st.beta[16 * I + rr];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * p + e;
    if (NEEDQ) st.aqk[I][i][rr] = static_cast<bf16>(rr <= i ? accq[e] : 0.f);
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

// Values of block I as the A operand of a 16x16x32 product: lane (r, p) holds token
// 16 I + r, the VW = 32 / (4 / NT) value columns cbase + VW p .. of this wavefront (NT = 2:
// 16 bytes; NT = 1: 8 bytes and four zeros). One row piece per lane instead of 4 NT
// two-byte loads in the accumulator layout; the product with a -1 selector (vsel) turns it
// into -V in the accumulator layout, onto which (K P) S accumulates.
template <int NT, int DV>
__device__ __forceinline__ bf16x8 load_vrow(rsrc_t v, uint32_t off) {
  if constexpr (NT == 2) return __builtin_bit_cast(bf16x8, ld_b128(v, off));
  else return cat8(ld_b64(v, off), bf16x4{});
}
// The selector of value tile c: B[8 p + i][r] = -1 where the lane's column VW p + i is the
// tile's column 16 c + r.
template <int NT>
__device__ __forceinline__ bf16x8 vsel(int c, int rr, int p) {
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    b[i] = static_cast<bf16>(i < 4 * NT && 4 * NT * p + i == 16 * c + rr ? -1.f : 0.f);
  return b;
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
//   kModeHist  the state entering every pair of blocks in a.hist (at byte hist_off, the
//              layout of hist_chain_offset), for the backward pass; no outputs;
//   kModeState nothing else (the end state of a segment started from zero);
//   kModeTrans the transition of the segment: the identity as initial state and zero values,
//              so that the final state is the dk x dk product of the segment's token maps;
//   kModeTransOut  the same, and its outputs: with the identity as state the output of token t
//              is the query carried back to the segment start (M_t^T q_t, M_t the product of
//              the token maps up to t), dk values per token, so that the output from any start
//              state S is S^T M_t^T q_t plus the output from the zero state.
// Outputs go to rows orow0 .. of obase (DV values per row).
template <int NT, int DV, bool GDR2, int MODE>
__device__ __forceinline__ void state_role(Smem& sm, const ChunkArgs& a, const TokenRange& tr,
                                           size_t row0, const float* s0p, float* sTp,
                                           size_t hist_off, int nsteps, int cbase, int lane,
                                           int rr, int p, void* obase, size_t orow0) {
  constexpr bool HIST = MODE == kModeHist;
  constexpr bool OUT = MODE == kModeOut || MODE == kModeTransOut;
  constexpr bool TRANS = MODE == kModeTrans || MODE == kModeTransOut;
  // (the transition reads no values: a zero-sized view returns zeros)
  const rsrc_t vsrc = make_rsrc(static_cast<const bf16*>(a.v) + row0 * DV,
                                TRANS ? 0u : (uint32_t)tr.len * DV * 2);
  const rsrc_t odst = make_rsrc(static_cast<bf16*>(obase) + (OUT ? orow0 * DV : 0),
                                OUT ? (uint32_t)tr.len * DV * 2 : 0u);
  const rsrc_t hdst = make_rsrc(static_cast<char*>(a.hist) + (HIST ? hist_off : 0),
                                HIST ? (uint32_t)nsteps * 2 * kDK * DV * 2 : 0);
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
  // (the transition reads no write gates either: its DV = dk may differ from their width)
  const rsrc_t wsrc = GDR2 ? make_rsrc(a.write + (TRANS ? 0 : row0 * DV),
                                       TRANS ? 0u : (uint32_t)tr.len * DV * 4)
                           : vsrc;
  // KDA: value row pieces of the four blocks (token 16 I + rr at vrow + I * 16 DV * 2 bytes)
  // and the selectors that turn them into -V; Gated Delta Rule-2: values and write gates in
  // the accumulator layout (w * V is formed on the vector ALU)
  constexpr bool VSEL = !GDR2;
  const uint32_t vrow = (uint32_t)(rr * DV + cbase + 4 * NT * p) * 2;
  bf16x8 va[4];
  bf16x8 sel[NT];
  bf16 vv[NT][4][4];
  float ww[NT][4][4];
  if constexpr (VSEL) {
#pragma unroll
    for (int c = 0; c < NT; ++c) sel[c] = vsel<NT>(c, rr, p);
    if constexpr (!TRANS) {
#pragma unroll
      for (int I = 0; I < 4; ++I) va[I] = load_vrow<NT, DV>(vsrc, vrow + I * 16 * DV * 2);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        load_values<DV>(vv[c][I], vsrc, voff[c] + I * 16 * DV * 2);
        if (GDR2) load_gates<DV>(ww[c][I], wsrc, 2 * (voff[c] + I * 16 * DV * 2));
      }
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
      // KDA: X starts as -V, so that the chain below leaves X - V
      if constexpr (VSEL && !TRANS) {
#pragma unroll
        for (int c = 0; c < NT; ++c) X[c] = mfma32(va[I], sel[c], X[c]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&st.kr[16 * I + rr][32 * ks + 8 * p]);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const bf16x8 sb = cat8(pack4(S_acc[c][2 * ks]), pack4(S_acc[c][2 * ks + 1]));
          X[c] = mfma32(ak, sb, X[c]);
          if constexpr (HIST) {
            if ((I & 1) == 0) {  // the state entering each pair of blocks
              const uint32_t tile = (uint32_t)(2 * s + I / 2) * (DV / 16) + (cbase + 16 * c) / 16;
              st_b128(hdst, ((tile * 4 + ks) * 64 + lane) * 16, sb);
            }
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
      if constexpr (VSEL) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          f32x4 R;
#pragma unroll
          for (int e = 0; e < 4; ++e) R[e] = -bt[e] * X[c][e];
          vp[c] = pack4(R);
        }
        if constexpr (!TRANS)  // the next 64 tokens' values of this block
          va[I] = load_vrow<NT, DV>(vsrc, vrow + cbyte + (I * 16 + kC) * DV * 2);
      } else {
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
          if (GDR2)
            load_gates<DV>(ww[c][I], wsrc, 2 * (voff[c] + cbyte + (I * 16 + kC) * DV * 2));
        }
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
  int kseg = 0, skind = kSegWhole;  // segment plans: segment index and item kind
  if constexpr (MODE == kModeSeg) {
    if (blockIdx.x >= a.plan[0]) return;  // the grid is sized for the largest plan
    const uint32_t* it = a.plan + segplan_items_off(a.N, a.seg_slots) + 2 * blockIdx.x;
    chain = (int)(it[0] >> 2);
    part = (int)(it[0] & 3);
    kseg = (int)(it[1] >> 2);
    skind = (int)(it[1] & 3);
    if (chain >= a.N * a.H) return;
  } else if (a.plan) {
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
  // segment plans: segment kseg of X tokens of its sequence. The first segment runs from the
  // chain's initial state and leaves the start state of the second; every later one runs
  // twice, from the zero state (outputs and end state) and as its transition (carried-back
  // queries and the dk x dk transition), and its outputs are completed afterwards.
  void* obase = a.o;
  size_t qrow = 0;  // transitions: the first row of the carried-back queries they write
  if constexpr (MODE == kModeSeg) {
    if (skind != kSegWhole) {
      const int xt = (int)a.plan[1] * kC;
      const int first = kseg * xt;
      if (xt <= 0 || first >= tr.len) return;
      tr.t0 += first;
      tr.len = min(xt, tr.len - first);
      const size_t slot = a.plan[kSegHdr + n] + (size_t)kseg;
      if (slot + 1 >= (size_t)a.seg_slots + (skind == kSegFirst ? 0 : 1)) return;
      const size_t msz = (size_t)kDK * DV, per = (size_t)a.seg_slots * a.H * msz;
      if (skind == kSegFirst) {
        sTp = a.seg_mats + ((slot + 1) * a.H + h) * msz;         // start of segment 1
      } else if (skind == kSegZero) {
        s0p = nullptr;
        sTp = a.seg_mats + 2 * per + (slot * a.H + h) * msz;     // B: end state from zero
      } else {
        s0p = nullptr;
        sTp = a.seg_mats + per + (slot * a.H + h) * msz;         // A: the transition
        obase = a.qt;                                            // Qt: rows of head h
        qrow = (size_t)h * a.plan[4] + a.plan[segplan_qoff_off(a.N, a.seg_slots) + slot];
      }
    }
  }
  const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0;
  const size_t orow0 = obase == a.o ? row0 : qrow;
  const size_t hist_off = HIST ? hist_chain_offset(a, n, h, tr) : 0;
  const int nsteps = (tr.len + kC - 1) / kC;

  if (prep_wave) {
    // ---------------- prep wavefront: block I of every 64 tokens (the state history pass
    // writes no outputs and forms no query operands)
    constexpr bool NEEDQ = MODE != kModeHist;
    const int I = wave;
    const PrepSrc src = prep_src<PER_CHANNEL, GDR2>(a, row0, tr.len, I, lane);
    BlockRegs r;
    if (nsteps > 0) {
      load_block<PER_CHANNEL, GDR2, NEEDQ>(r, src, 0);
      prep_block<GDR2, NEEDQ>(sm.st[0], sm.kd, r, I, lane);
      wave_lds_fence();
      block_tiles<NEEDQ>(sm.st[0], sm.kd, I, rr, p);
      if (nsteps > 1) load_block<PER_CHANNEL, GDR2, NEEDQ>(r, src, kC);
    }
    lds_barrier();
    for (int s = 0; s < nsteps; ++s) {
      if (s + 1 < nsteps) {
        Stage& st = sm.st[(s + 1) & 1];
        prep_block<GDR2, NEEDQ>(st, sm.kd, r, I, lane);
        wave_lds_fence();
        block_tiles<NEEDQ>(st, sm.kd, I, rr, p);
        if (s + 2 < nsteps) load_block<PER_CHANNEL, GDR2, NEEDQ>(r, src, (s + 2) * kC);
      }
      lds_barrier();
    }
  } else {
    // ---------------- state wavefront
    // The state steps are the sequential critical path; with the Gated Delta Rule-2 gates
    // or one decay per head they take issue priority over the prep wavefronts sharing a
    // SIMD (the KDA gates measured fastest at equal priority, see KDA_STATE_PRIO_KDA).
    constexpr short kStatePrio = PER_CHANNEL && !GDR2 ? KDA_STATE_PRIO_KDA : KDA_STATE_PRIO;
    __builtin_amdgcn_s_setprio(kStatePrio);
    const int j = wave - kPrepWaves;
    if constexpr (MODE == kModePair) {  // whole items only
      if (kind == kModeTrans)
        state_role<NT, DV, GDR2, kModeTrans>(sm, a, tr, row0, s0p, sTp, 0, nsteps, 16 * NT * j,
                                             lane, rr, p, nullptr, 0);
      else
        state_role<NT, DV, GDR2, kModeState>(sm, a, tr, row0, s0p, sTp, 0, nsteps, 16 * NT * j,
                                             lane, rr, p, nullptr, 0);
      return;
    }
    // segment plans: the transition items, then whole or half output items
    constexpr int RMODE = MODE == kModeSeg ? kModeOut : MODE;
    if constexpr (MODE == kModeSeg) {
      if (skind == kSegTrans) {
        state_role<NT, DV, GDR2, kModeTransOut>(sm, a, tr, row0, s0p, sTp, 0, nsteps,
                                                16 * NT * j, lane, rr, p, obase, orow0);
        return;
      }
    }
    if constexpr (NT > 1) {
      if (part) {  // a half item: NT / 2 tiles per wavefront over one half of the columns
        state_role<NT / 2, DV, GDR2, RMODE>(sm, a, tr, row0, s0p, sTp, hist_off, nsteps,
                                            (part == 2 ? DV / 2 : 0) + 16 * (NT / 2) * j, lane,
                                            rr, p, obase, orow0);
        return;
      }
    }
    state_role<NT, DV, GDR2, RMODE>(sm, a, tr, row0, s0p, sTp, hist_off, nsteps, 16 * NT * j,
                                    lane, rr, p, obase, orow0);
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

// ---------------------------------------------------------------------------------------
// Segment plan. The schedule above cannot shorten a chain below kHalfCost of its length; when
// the longest sequences still bound the launch, they are cut into segments of X tokens
// instead. The first segment runs as usual from the initial state and hands its end state to
// the second; every later segment k runs twice at the same time as the others, from the zero
// state (outputs O0 and end state B_k) and from the identity (its dk x dk transition A_k and
// the carried-back queries Qt). By linearity in the start state S_k, the segment's outputs
// are O0 + Qt S_k and its end state A_k S_k + B_k: a short chain over the segments gives
// every S_k (seg_chain_kernel) and a matrix-core pass adds Qt S_k (seg_correct_kernel).
// The planner picks X (a multiple of 64 tokens, at least xc_min chunks) to minimise
// max(longest item, total work / compute units) plus the cost of the corrections; without a
// gain of kSegMinGain it keeps the halves schedule. Chunk counts stand for item times.

constexpr int kSegGroup = 256;           // tokens per correction unit
// (measured on MI355X, one chunk-time = 64 tokens of one item, about 4.5 us)
constexpr float kSegCorrCost = 0.4f;     // correction of one chunk, in chunk-times of one item
constexpr float kSegFixedCost = 8.f;     // the planner's extra time and the two extra launches
constexpr float kSegChainCost = 0.5f;    // one step of the chain over the segments
constexpr float kSegPacking = 1.1f;      // list scheduling of items shorter than the longest
constexpr float kSegMinGain = 0.95f;

// bitonic sort of entries 0 .. n2 - 1 (n2 a power of two, at most the block size): larger
// key first, then lower (a, b)
__device__ __forceinline__ void sort_entries(int* key, int* ea, int* eb, int n2) {
  const int t = threadIdx.x;
  for (int k = 2; k <= n2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int u = t ^ j;
      if (t < n2 && u > t) {
        const bool t_first =
            key[t] > key[u] ||
            (key[t] == key[u] && (ea[t] < ea[u] || (ea[t] == ea[u] && eb[t] < eb[u])));
        if (((t & k) == 0) != t_first) {
          const int k0 = key[t], a0 = ea[t], b0 = eb[t];
          key[t] = key[u];
          ea[t] = ea[u];
          eb[t] = eb[u];
          key[u] = k0;
          ea[u] = a0;
          eb[u] = b0;
        }
      }
      __syncthreads();
    }
}

// Exclusive prefix sum of v over the BS threads of the block (every thread calls it with its
// value; x is BS + 1 words of scratch): returns the sum over lower threads and leaves the
// total in x[BS]. Wavefront scans by lane shifts, then the wavefront totals.
template <int BS>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* x) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  __syncthreads();  // earlier readers of x are done
  if (lane == 63) x[wv] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
  for (int i = 0; i < BS / 64; ++i) {
    const uint32_t wt = x[i];
    if (i < wv) before += wt;
    total += wt;
  }
  __syncthreads();
  if (t == 0) x[BS] = total;
  __syncthreads();
  return before + incl - v;
}

// The plan is laid out for slots_max slots (the workspace's capacity); a candidate segment
// length is allowed only when its slots fit that capacity (and mats_ok: the workspace holds
// the matrices of every slot) and its carried-back queries fit qt_rows rows per head.
// xc_max > 0 bounds every item to xc_max chunks: sequences longer than that are always cut
// (the host has checked that a candidate within the bound fits the workspace).
// BS threads (256 or 1024) plan up to BS sequences into up to BS slots, with BS candidates.
template <int BS>
__global__ __launch_bounds__(BS) void chunk_segplan_kernel(
    const int32_t* cu, int N, int H, int T, int cus, int slots_max, int mats_ok,
    long long qt_rows, int xc_min, int xc_max, uint32_t* plan) {
  __shared__ int cl[BS];     // chunks of sequence n
  __shared__ int ln[BS];     // tokens of sequence n
  __shared__ int key[BS];    // entries: chunks
  __shared__ int ea[BS];     //          sequence
  __shared__ int eb[BS];     //          segment
  __shared__ float bnd[BS];  // bound of candidate segment length j
  __shared__ int bix[BS];
  __shared__ int ent_parts[BS];
  __shared__ uint32_t ent_off[BS + 1];
  __shared__ int n_ent, xc_sel;
  const int t = threadIdx.x;
  uint32_t* segbase = plan + kSegHdr;
  uint32_t* corr_off = plan + segplan_corr_off(N);
  uint32_t* qoff = plan + segplan_qoff_off(N, slots_max);
  uint32_t* items = plan + segplan_items_off(N, slots_max);
  int c = -1;
  if (t < N) {
    const int len = token_range(cu, t, T).len;
    c = (len + kC - 1) / kC;
    cl[t] = c;
    ln[t] = len;
  }
  key[t] = c;
  ea[t] = t;
  eb[t] = 0;
  __syncthreads();
  int n2 = 1;
  while (n2 < N) n2 <<= 1;
  sort_entries(key, ea, eb, n2);
  const int maxc = key[0] > 0 ? key[0] : 0;
  // sequences past the item bound must be cut
  const bool must_cut = xc_max > 0 && maxc > xc_max;
  // candidate segment lengths xc_min + j * step (chunks), shorter than the longest sequence
  // and within the item bound
  const int hi = must_cut ? xc_max + 1 : maxc;
  const int step = hi > xc_min ? (hi - xc_min + BS - 1) / BS : 1;
  {
    const int xc = xc_min + t * step;
    float b = 3.0e38f;
    if (mats_ok && xc < hi) {
      long long total = 0, corr = 0, slots = 0, later = 0;
      int longest = 0, most = 1;
      for (int i = 0; i < N; ++i) {
        const int ci = cl[i];
        const int extra = ci > xc ? ci - xc : 0;
        const int ns_i = ci > xc ? (ci + xc - 1) / xc : 1;
        slots += ns_i;
        most = max(most, ns_i);
        total += ci + extra;
        corr += extra;
        later += ci > xc ? ln[i] - xc * kC : 0;  // tokens past the first segment
        longest = max(longest, min(ci, xc));
      }
      if (slots <= slots_max && slots <= BS && later <= qt_rows)
        b = fmaxf((float)longest, kSegPacking * H * total / cus) +
            kSegCorrCost * H * corr / cus + kSegFixedCost + kSegChainCost * (most - 1);
    }
    bnd[t] = b;
    bix[t] = t;
  }
  __syncthreads();
  {  // the best candidate (lowest index on ties): within each wavefront, then across them
    float bv = bnd[t];
    int bi = t;
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
      const float ov = __shfl_xor(bv, d, 64);
      const int oi = __shfl_xor(bi, d, 64);
      if (ov < bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    __syncthreads();
    if ((t & 63) == 0) {
      bnd[t >> 6] = bv;
      bix[t >> 6] = bi;
    }
    __syncthreads();
    if (t == 0) {
      for (int i = 1; i < BS / 64; ++i)
        if (bnd[i] < bnd[0] || (bnd[i] == bnd[0] && bix[i] < bix[0])) {
          bnd[0] = bnd[i];
          bix[0] = bix[i];
        }
    }
    __syncthreads();
  }
  if (t == 0) {
    // the halves schedule (as chunk_plan_kernel) and its bound, in fp32 (chunk counts times
    // H stay far below 2^24 per sequence; the sums only rank schedules)
    const float rcus = 1.f / (float)cus, hc = (float)kHalfCost;
    float total = 0.f;
    for (int i = 0; i < N; ++i) total += (float)key[i] * (float)H;
    int ns = 0;
    float maxhalf = 0.f;
    while (ns < N && key[ns] > 0) {
      const float c0 = (float)key[ns], next = ns + 1 < N ? (float)key[ns + 1] : 0.f;
      const float bound = fmaxf(fmaxf(c0, maxhalf), total * rcus);
      const float total2 = total + (float)H * (2.f * hc - 1.f) * c0;
      const float maxhalf2 = fmaxf(maxhalf, hc * c0);
      if (!(fmaxf(fmaxf(next, maxhalf2), total2 * rcus) < 0.98f * bound)) break;
      total = total2;
      maxhalf = maxhalf2;
      ++ns;
    }
    const float half_bound = fmaxf(fmaxf(ns < N ? (float)key[ns] : 0.f, maxhalf), total * rcus);
    const bool any = bnd[0] < 3.0e38f;
    xc_sel = any && (must_cut || bnd[0] < kSegMinGain * half_bound) ? xc_min + bix[0] * step : 0;
    plan[1] = (uint32_t)xc_sel;
    if (must_cut && xc_sel == 0) {
      // no candidate fits (the host rules this out): an empty plan, no item runs
      n_ent = 0;
      ent_off[0] = 0;
      plan[0] = plan[2] = plan[3] = plan[4] = 0;
    } else if (xc_sel == 0) {
      // the halves schedule: sequences by chunk count, halves of the ns longest
      int a = 0, b = ns, e = 0;
      uint32_t off = 0;
      while (a < ns || b < N) {
        const bool split = a < ns && (b >= N || kHalfCost * key[a] >= key[b]);
        const int i = split ? a++ : b++;
        eb[e] = ea[i];  // the merge reads key and ea only
        ent_parts[e] = split ? 2 : 1;
        ent_off[e] = off;
        off += (uint32_t)H * ent_parts[e];
        ++e;
      }
      ent_off[e] = off;
      n_ent = e;
      plan[0] = off;
      plan[2] = 0;
      plan[3] = 0;
      plan[4] = 0;
    }
  }
  __syncthreads();
  const int xc = xc_sel;
  if (xc == 0) {
    if (t < n_ent) ea[t] = eb[t];
    __syncthreads();
  } else {
    // segments of every sequence, in sequence order (slot = segbase[n] + k)
    const int ns_t = t < N ? (cl[t] > xc ? (cl[t] + xc - 1) / xc : 1) : 0;
    const uint32_t base = block_exclusive_scan<BS>((uint32_t)ns_t, ent_off);
    const int slots = (int)ent_off[BS];
    if (t < N) {
      segbase[t] = base;
      for (int k = 0; k < ns_t; ++k) {
        key[base + k] = ns_t == 1 ? cl[t] : min(xc, cl[t] - k * xc);
        ea[base + k] = t;
        eb[base + k] = k;
      }
    }
    if (t == 0) segbase[N] = (uint32_t)slots;
    if (t >= slots) key[t] = -1;  // padding sorts last
    __syncthreads();
    // correction units of every slot (later segments only), in slot order
    uint32_t units = 0;
    if (t < slots && eb[t] > 0) {
      const int len = ln[ea[t]], k = eb[t];
      units = (uint32_t)(min(xc * kC, len - k * xc * kC) + kSegGroup - 1) / kSegGroup;
    }
    const uint32_t uoff = block_exclusive_scan<BS>(units, ent_off);
    if (t < slots) corr_off[t] = uoff;
    if (t == 0) {
      corr_off[slots] = ent_off[BS];
      plan[2] = (uint32_t)slots;
      plan[3] = ent_off[BS];
    }
    // rows of carried-back queries of every slot (later segments only), in slot order
    uint32_t qrows = 0;
    if (t < slots && eb[t] > 0) {
      const int len = ln[ea[t]], k = eb[t];
      qrows = (uint32_t)min(xc * kC, len - k * xc * kC);
    }
    const uint32_t qo = block_exclusive_scan<BS>(qrows, ent_off);
    if (t < slots) qoff[t] = qo;
    if (t == 0) {
      qoff[slots] = ent_off[BS];
      plan[4] = ent_off[BS];
    }
    __syncthreads();
    int m2 = 1;
    while (m2 < slots) m2 <<= 1;
    sort_entries(key, ea, eb, m2);
    // items of every entry: whole sequences and first segments H, later segments 2 H
    int parts = 0;
    if (t < slots) {
      const int n = ea[t];
      const bool split = cl[n] > xc;
      parts = !split ? 0 : eb[t] == 0 ? 1 : 2;
      ent_parts[t] = parts;
    }
    const uint32_t eoff = block_exclusive_scan<BS>(t < slots ? (uint32_t)H * (parts == 2 ? 2 : 1) : 0u,
                                               ent_off);
    const uint32_t tot = ent_off[BS];
    __syncthreads();
    if (t < slots) ent_off[t] = eoff;
    if (t == 0) {
      ent_off[slots] = tot;
      n_ent = slots;
      plan[0] = tot;
    }
    __syncthreads();
  }
  const uint32_t n_items = ent_off[n_ent];
  for (uint32_t i = t; i < n_items; i += BS) {
    int lo = 0, hi = n_ent - 1;  // entry holding item i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ent_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const uint32_t local = i - ent_off[lo];
    uint32_t hh = local, part = 0, w1 = 0;
    if (xc == 0) {
      if (ent_parts[lo] == 2) split_item(local, (uint32_t)H, hh, part);
    } else {
      const int kind = ent_parts[lo] == 0 ? kSegWhole
                       : ent_parts[lo] == 1 ? kSegFirst
                       : (local < (uint32_t)H ? kSegZero : kSegTrans);
      hh = local % (uint32_t)H;
      w1 = ((uint32_t)eb[lo] << 2) | (uint32_t)kind;
    }
    items[2 * i] = (((uint32_t)ea[lo] * H + hh) << 2) | part;
    items[2 * i + 1] = w1;
  }
}

template <int NS, int NT, bool PER_CHANNEL, int MODE>
hipError_t launch_ns(const ChunkArgs& a, unsigned grid, hipStream_t stream) {
  if constexpr (MODE == kModeOut || MODE == kModeHist || MODE == kModeState ||
                MODE == kModeTrans) {
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
hipError_t launch_mode(const ChunkArgs& args, bool per_channel, int dv, hipStream_t stream,
                       bool build_plan = true) {
  ChunkArgs a = args;
  const bool can_split = dv == 128;  // a half of dv = 128 is one 16-column tile per wavefront
  const long long items =
      (long long)a.N * a.H * (a.seg_len > 0 ? a.nseg : 1) * (MODE == kModePair ? 2 : 1);
  unsigned grid = (unsigned)items;
  a.split_all = 0;
  if (a.plan && a.cu && a.seg_len == 0) {
    // packed sequences: the work list is built on the device from cu_seqlens
    if (build_plan) {
      chunk_plan_kernel<<<1, kMaxPlanSeqs, 0, stream>>>(a.cu, a.N, a.H, a.T, a.cus, can_split,
                                                        a.plan);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
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

// S_{k+1} = A_k S_k + B_k over the segments of every sequence cut into three or more (fp32
// matrix cores), from the second segment's start state (which the first segment's item
// writes): the start state of every later segment. The last step, to the final state, is
// taken by seg_correct_kernel beside the output corrections, so that sequences cut in two
// (the common case) need no step here. One workgroup of eight
// wavefronts per (chain, 16 value columns), so that chains with many segments spread each
// step over many compute units; wavefront w owns rows 16 w .. 16 w + 15. A lane holds the
// operands of two steps, the current one and the next one in flight (92 registers, two
// workgroups per compute unit). Most workgroups belong to uncut chains and leave after one
// load; with few of them resident at once they would pass through the device in rounds.
__global__ __launch_bounds__(512) void seg_chain_kernel(ChunkArgs a) {
  __shared__ __align__(16) float St[16][kDK + 4];  // S^T: [column][row]
  const uint32_t* plan = a.plan;
  const int chain = blockIdx.x, cb = 16 * blockIdx.y;
  const int n = chain / a.H, h = chain % a.H;
  // the plan's flag and the sequence's slots, loaded together
  const uint32_t on = plan[1], s0 = plan[kSegHdr + n], s1 = plan[kSegHdr + n + 1];
  const uint32_t ns = s1 - s0;
  if (on == 0 || s1 < s0 || ns < 3 || s1 > (uint32_t)a.seg_slots) return;
  const uint32_t kend = ns - 1;  // steps 1 .. kend - 1 write the start states 2 .. kend
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, rr = lane & 15, p = lane >> 4;
  const size_t msz = (size_t)kDK * kDK, per = (size_t)a.seg_slots * a.H * msz;
  const float* first = a.seg_mats + ((size_t)(s0 + 1) * a.H + h) * msz;
  for (int i = threadIdx.x; i < kDK * 16; i += 512)
    St[i & 15][i >> 4] = first[(size_t)(i >> 4) * kDK + cb + (i & 15)];
  // operands of step k: A[16 wv + rr][4 p + 16 j .. + 3] (16-byte loads) and
  // B[16 wv + 4 p + e][cb + rr]; product (j, e) contracts channel 4 p + 16 j + e of lane
  // group p, whose S entries for e = 0 .. 3 are one 16-byte read of the transposed tile
  f32x4 x0[8], x1[8], y0, y1;
  auto load = [&](uint32_t k, f32x4 (&x)[8], f32x4& y) {
    const size_t m = ((size_t)(s0 + k) * a.H + h) * msz;
    const float* Ar = a.seg_mats + per + m + (size_t)(16 * wv + rr) * kDK + 4 * p;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = *reinterpret_cast<const f32x4*>(Ar + 16 * j);
    const float* Br = a.seg_mats + 2 * per + m + (size_t)(16 * wv + 4 * p) * kDK + cb + rr;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = Br[(size_t)e * kDK];
  };
  auto step = [&](uint32_t k, const f32x4 (&x)[8], const f32x4& y) {
    __syncthreads();  // S of step k is in LDS
    f32x4 acc = y;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 sb = *reinterpret_cast<const f32x4*>(&St[rr][4 * p + 16 * j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma_f32(x[j][e], sb[e], acc);
    }
    __syncthreads();  // every read of S is done
    float* dst = a.seg_mats + ((size_t)(s0 + k + 1) * a.H + h) * msz;
    *reinterpret_cast<f32x4*>(&St[rr][16 * wv + 4 * p]) = acc;  // rows 16 wv + 4 p + e
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(size_t)(16 * wv + 4 * p + e) * kDK + cb + rr] = acc[e];
  };
  // two register sets: step k + 1's operands are in flight during step k
  load(1, x0, y0);
  if (2 < kend) load(2, x1, y1);
  for (uint32_t k = 1; k < kend; k += 2) {
    step(k, x0, y0);
    if (k + 2 < kend) load(k + 2, x0, y0);
    if (k + 1 < kend) {
      step(k + 1, x1, y1);
      if (k + 3 < kend) load(k + 3, x1, y1);
    }
  }
}

// Outputs of the later segments of a segment plan: O += Qt S_k, one unit of kSegGroup tokens
// of one segment and head per pass of a workgroup. S_k^T is staged in LDS as the bf16 A
// operands of its eight 16-column tiles; wavefront w takes 16-token blocks w, w + 4, ...,
// with the queries as the B operand, so that each product is a tile of O^T. The fp32 sums
// go through a wavefront-private LDS tile, and O is read and written as whole 256-byte
// rows (16 bytes per lane). The next block's loads are issued before the current block's
// products. The same launch takes the last step of every cut sequence's segment chain,
// S_T = A S + B from the last segment's start state, one unit per (sequence, 16 value
// columns, head), after the corrections: small matrix-core products in the tail of their
// memory-bound passes, instead of a launch of their own.
constexpr int kCorrLd = kDK + 4;  // padded row (floats) of the correction tile
__device__ __forceinline__ bf16x8 to_bf16x8_(const float (&x)[8]) {
  return cat8(pack4(x[0], x[1], x[2], x[3]), pack4(x[4], x[5], x[6], x[7]));
}
__global__ __launch_bounds__(256) void seg_correct_kernel(ChunkArgs a) {
  __shared__ bf16x8 sa[8][4][64];            // [column tile][32-channel slab][lane]
  __shared__ __align__(16) float ct_[4][16][kCorrLd];  // per wavefront: 16 tokens x 128 columns
  __shared__ uint32_t segbase[kMaxPlanSeqs + 1], corr_off[kMaxPlanSeqs + 1];
  __shared__ uint32_t cut[kMaxPlanSeqs], scan_x[257];  // the sequences cut in two or more
  const uint32_t* plan = a.plan;
  const uint32_t units = plan[3], slots = plan[2];
  if (plan[1] == 0 || units == 0 || slots == 0 || slots > (uint32_t)a.seg_slots ||
      slots > (uint32_t)kMaxPlanSeqs || a.N > kMaxPlanSeqs)
    return;
  for (int i = threadIdx.x; i <= a.N; i += 256) segbase[i] = plan[kSegHdr + i];
  for (uint32_t i = threadIdx.x; i <= slots; i += 256) corr_off[i] = plan[segplan_corr_off(a.N) + i];
  __syncthreads();
  // the cut sequences in order (thread t looks at sequences 4 t .. 4 t + 3)
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = 4 * (int)threadIdx.x + i;
    if (n < a.N && segbase[n + 1] >= segbase[n] + 2) ++mine;
  }
  uint32_t at = block_exclusive_scan<256>(mine, scan_x);
  const uint32_t ncut = scan_x[256];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = 4 * (int)threadIdx.x + i;
    if (n < a.N && segbase[n + 1] >= segbase[n] + 2) cut[at++] = (uint32_t)n;
  }
  __syncthreads();
  const int xt = (int)plan[1] * kC;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rr = lane & 15, p = lane >> 4;
  const size_t msz = (size_t)kDK * kDK;
  float (*cw)[kCorrLd] = ct_[wv];
  const uint32_t qt_per_head = plan[4];  // rows of carried-back queries per head
  // units: the corrections, then the final states (when requested)
  const uint32_t nfin = a.sT ? ncut * 8u * (uint32_t)a.H : 0u;
  const uint32_t ncorr = units * (uint32_t)a.H;
  for (uint32_t w0 = blockIdx.x; w0 < nfin + ncorr; w0 += gridDim.x) {
    if (w0 >= ncorr) {
      const uint32_t w = w0 - ncorr;
      // S_T = A S + B for 16 value columns of one chain, from the start state of its
      // sequence's last segment; wavefront wv owns row tiles 2 wv and 2 wv + 1, A rows in
      // registers (16-byte loads), S^T of the columns through LDS (ct_[0], free between units)
      const int h = (int)(w % (uint32_t)a.H);
      const int cb = 16 * (int)((w / (uint32_t)a.H) % 8u);
      const uint32_t n = cut[w / (8u * (uint32_t)a.H)];
      const uint32_t sl = segbase[n + 1] - 1;  // the last segment's slot
      const size_t pm = (size_t)a.seg_slots * a.H * msz;
      const float* Sk = a.seg_mats + ((size_t)sl * a.H + h) * msz;
      f32x4 xa[2][8], acc[2];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int r0 = 16 * (2 * wv + ti);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          xa[ti][j] = *reinterpret_cast<const f32x4*>(Sk + pm + (size_t)(r0 + rr) * kDK + 4 * p +
                                                      16 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[ti][e] = Sk[2 * pm + (size_t)(r0 + 4 * p + e) * kDK + cb + rr];
      }
      float sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = (int)threadIdx.x + 256 * i;
        sv[i] = Sk[(size_t)(idx >> 4) * kDK + cb + (idx & 15)];
      }
      float (*St)[kCorrLd] = ct_[0];  // St[c][r] = S[r][cb + c]
      __syncthreads();  // earlier readers of ct_ are done
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = (int)threadIdx.x + 256 * i;
        St[idx & 15][idx >> 4] = sv[i];
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 sb = *reinterpret_cast<const f32x4*>(&St[rr][4 * p + 16 * j]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int ti = 0; ti < 2; ++ti) acc[ti] = mfma_f32(xa[ti][j][e], sb[e], acc[ti]);
      }
      float* dst = a.sT + ((size_t)n * a.H + h) * msz;
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[(size_t)(16 * (2 * wv + ti) + 4 * p + e) * kDK + cb + rr] = acc[ti][e];
      continue;
    }
    const int h = (int)(w0 % (uint32_t)a.H);
    const uint32_t u = w0 / (uint32_t)a.H;
    uint32_t lo = 0, hi = slots - 1;  // the last slot whose first unit is <= u
    while (lo < hi) {
      const uint32_t mid = (lo + hi + 1) >> 1;
      if (corr_off[mid] <= u) lo = mid; else hi = mid - 1;
    }
    // the searches read LDS, so their results sit in vector registers; they are the same in
    // every lane, and as scalars the unit's buffer descriptors need no loop over lanes
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lo);
    int nlo = 0, nhi = a.N - 1;  // the sequence of slot sl
    while (nlo < nhi) {
      const int mid = (nlo + nhi + 1) >> 1;
      if (segbase[mid] <= sl) nlo = mid; else nhi = mid - 1;
    }
    const int n = __builtin_amdgcn_readfirstlane(nlo);
    const int k = (int)(sl - __builtin_amdgcn_readfirstlane(segbase[n]));
    const TokenRange tr = token_range(a.cu, n, a.T);
    const int g0 = k * xt + (int)(u - __builtin_amdgcn_readfirstlane(corr_off[sl])) *
                                kSegGroup;  // first token of the unit
    const int seg_end = (int)min((long long)(k + 1) * xt, (long long)tr.len);
    if (k < 1 || g0 >= seg_end) continue;  // uniform over the workgroup
    const int len = min(kSegGroup, seg_end - g0);
    const size_t row0 = ((size_t)tr.b * a.H + h) * a.T + tr.t0 + g0;
    // the unit's carried-back queries: rows of head h from the slot's first row
    const size_t qrow0 =
        (size_t)h * qt_per_head +
        __builtin_amdgcn_readfirstlane(plan[segplan_qoff_off(a.N, a.seg_slots) + sl]) +
        (size_t)(g0 - k * xt);
    const rsrc_t qs = make_rsrc(static_cast<const bf16*>(a.qt) + qrow0 * kDK, (uint32_t)len * kDK * 2);
    const rsrc_t os = make_rsrc(static_cast<bf16*>(a.o) + row0 * kDK, (uint32_t)len * kDK * 2);
    const float* S = a.seg_mats + ((size_t)sl * a.H + h) * msz;
    // S^T staged as bf16: wavefront wv stages slab wv of every column tile; all 64 loads are
    // issued before the first wait
    float x[8][8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[ct][j] = S[(size_t)(32 * wv + 8 * p + j) * kDK + 16 * ct + rr];
    __syncthreads();  // the previous unit's reads of sa are done
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      sa[ct][wv][lane] = cat8(pack4(x[ct][0], x[ct][1], x[ct][2], x[ct][3]),
                              pack4(x[ct][4], x[ct][5], x[ct][6], x[ct][7]));
    __syncthreads();
    // block b0: queries of token b0 + rr (B operands), O rows as 16-byte pieces
    // (piece lane + 64 i: token b0 + piece / 16, columns 8 (piece % 16) ..)
    bf16x8 qb[4], ob[4];
    auto load = [&](int b0) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qb[ks] = __builtin_bit_cast(bf16x8, ld_b128(qs, (uint32_t)((b0 + rr) * kDK + 32 * ks + 8 * p) * 2));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pc = lane + 64 * i;
        ob[i] = __builtin_bit_cast(bf16x8, ld_b128(os, (uint32_t)((b0 + (pc >> 4)) * kDK + 8 * (pc & 15)) * 2));
      }
    };
    int b0 = 16 * wv;
    if (b0 < len) load(b0);
    for (; b0 < len; b0 += 64) {
      bf16x8 q_[4], o_[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q_[i] = qb[i];
        o_[i] = ob[i];
      }
      if (b0 + 64 < len) load(b0 + 64);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        f32x4 d = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) d = mfma32(sa[ct][ks][lane], q_[ks], d);
        // d[e] = correction of token b0 + rr, column 16 ct + 4 p + e
        *reinterpret_cast<f32x4*>(&cw[rr][16 * ct + 4 * p]) = d;
      }
      wave_lds_fence();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pc = lane + 64 * i, t = pc >> 4, c8 = 8 * (pc & 15);
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(&cw[t][c8]);
        const f32x4 c1 = *reinterpret_cast<const f32x4*>(&cw[t][c8 + 4]);
        float y[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = static_cast<float>(o_[i][e]) + c0[e];
          y[4 + e] = static_cast<float>(o_[i][4 + e]) + c1[e];
        }
        st_b128(os, (uint32_t)((b0 + t) * kDK + c8) * 2, to_bf16x8_(y));
      }
      wave_lds_fence();  // the tile is rewritten by the next block
    }
  }
}

}  // namespace

bool chunk_mfma_dims(int dk, int dv) { return dk == kDK && (dv == 64 || dv == 128); }

// Buffer descriptors address at most 2^31 bytes: a chain's g rows (T x dk fp32) must fit.
bool chunk_mfma_supports(int dk, int dv, int T) {
  return chunk_mfma_dims(dk, dv) && (long long)T * kDK * 4 < (1ll << 31);
}

// Longer chains run only as segment plans whose items are at most kMaxItemTokens long.
constexpr int kMaxItemTokens = 1 << 21;
static bool segplan_long(int T) { return !chunk_mfma_supports(kDK, kDK, T); }

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

// Segment plans: the shortest segment (64-token chunks), at least 512 tokens and at most 64
// segments per T tokens (within the item bound), and the most slots any candidate of the
// planner can use.
static int segplan_xc_min(int T) {
  const int ct = (int)(((long long)T + kC - 1) / kC);
  return std::min(kMaxItemTokens / kC, std::max(8, (ct + 63) / 64));
}
static int segplan_slots(int N, int T) {
  const int ct = (int)(((long long)T + kC - 1) / kC);
  return std::min(kMaxPlanSeqs, N + N / 8 + (ct + segplan_xc_min(T) - 1) / segplan_xc_min(T) + 1);
}
// Bytes of the plan words for a capacity of cap slots (up to 2 H items per slot).
static size_t segplan_plan_bytes(int N, int H, int cap) {
  return (4 * (segplan_items_off(N, cap) + 4 * (size_t)H * cap) + 255) / 256 * 256;
}
static size_t segplan_mats_bytes(int H, int cap) { return (size_t)3 * cap * H * kDK * kDK * 4; }

// Chains too long for whole-chain items: the slots and carried-back-query rows per head that
// a plan needs at the least. The planner's largest candidate within the item bound is at
// least 0.99 kMaxItemTokens long (its candidates are at most 129 chunks apart), so with
// m = ceil(T / kMaxItemTokens) >= 2, N packed sequences of T tokens in all take at most
// 2 N + 2 m slots and N sequences of T tokens each at most 2 m slots apiece; every token past
// a first segment needs a row.
static long long segplan_long_slots(int N, int T, bool packed) {
  if (!segplan_long(T)) return 0;
  const long long m = ((long long)T + kMaxItemTokens - 1) / kMaxItemTokens;
  return (packed ? 2ll * N + 2 * m : 2 * m * N) + 1;
}
static long long segplan_long_rows(int N, int T, bool packed) {
  return segplan_long(T) ? (packed ? (long long)T : (long long)N * T) : 0;
}

// Slots worth planning for: every sequence plus about one extra segment per compute unit and
// head (cutting beyond that only adds rounds of items), and what long chains need.
static int segplan_cap(int N, int H, int T, int cus, bool packed) {
  const long long need = segplan_long_slots(N, T, packed);
  return (int)std::max<long long>(
      need, std::max(N, std::min(segplan_slots(N, T), N + (cus + H - 1) / H + 1)));
}

// Layout of a segment plan in ws_bytes of workspace: the slot capacity (up to segplan_cap
// slots whose plan words and matrices fit, at least N so that the halves work list always
// fits), whether the matrices fit at all, and the rows of carried-back queries per head that
// the rest holds.
struct SegLayout {
  int cap = 0;
  bool mats_ok = false;
  long long qt_rows = 0;
};
// Chains too long for whole-chain items need the matrices of at least segplan_long_slots
// slots and segplan_long_rows rows, which are set aside first.
static bool segplan_layout(int N, int H, int T, int cus, bool packed, size_t ws_bytes,
                           SegLayout& L) {
  if (N <= 0 || N > kMaxPlanSeqs || H <= 0 || ws_bytes < segplan_plan_bytes(N, H, N)) return false;
  const long long need = segplan_long_slots(N, T, packed);
  if (need > kMaxPlanSeqs) return false;
  const size_t rows = (size_t)segplan_long_rows(N, T, packed) * H * kDK * 2;
  L = SegLayout{};
  L.cap = N;
  for (int cap = segplan_cap(N, H, T, cus, packed); cap >= std::max<long long>(N, need); --cap) {
    if (segplan_plan_bytes(N, H, cap) + segplan_mats_bytes(H, cap) + rows <= ws_bytes) {
      L.cap = cap;
      L.mats_ok = true;
      break;
    }
  }
  if (L.mats_ok) {
    const size_t used = segplan_plan_bytes(N, H, L.cap) + segplan_mats_bytes(H, L.cap);
    L.qt_rows = (long long)((ws_bytes - used) / ((size_t)H * kDK * 2));
  }
  return L.mats_ok || need == 0;
}

size_t chunk_segplan_min_bytes(int N, int H, int T, int dv, bool packed) {
  if (dv != kDK || N <= 0 || N > kMaxPlanSeqs || H <= 0) return 0;
  const long long need = segplan_long_slots(N, T, packed);
  if (need == 0) return segplan_plan_bytes(N, H, N);
  if (need > kMaxPlanSeqs) return 0;
  return segplan_plan_bytes(N, H, (int)need) + segplan_mats_bytes(H, (int)need) +
         (size_t)segplan_long_rows(N, T, packed) * H * kDK * 2;
}

// The workspace kda_chunk_fwd_workspace_size recommends: segplan_cap slots, and carried-back
// queries for the whole T axis of every sequence when the chains are fewer than the compute
// units (every sequence is then cut), else for a quarter of it (only the sequences much
// longer than the average are cut).
size_t chunk_segplan_bytes(int N, int H, int T, int dv, bool packed, int cus) {
  if (chunk_segplan_min_bytes(N, H, T, dv, packed) == 0) return 0;
  const int cap = segplan_cap(N, H, T, cus, packed);
  const long long chains = (long long)N * H;
  const long long rows = chains < cus || segplan_long(T)
                             ? (packed ? (long long)T : (long long)N * T)
                             : ((long long)T + 3) / 4;
  return segplan_plan_bytes(N, H, cap) + segplan_mats_bytes(H, cap) +
         (size_t)rows * H * kDK * 2;
}

hipError_t launch_chunk_mfma_segplan(const ChunkArgs& args, bool per_channel, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  ChunkArgs a = args;
  SegLayout L;
  if (!chunk_mfma_dims(a.dk, a.dv) || a.dv != kDK || !ws ||
      !segplan_layout(a.N, a.H, a.T, a.cus, a.cu != nullptr, ws_bytes, L))
    return hipErrorInvalidValue;
  const int sm = L.cap;
  a.plan = static_cast<uint32_t*>(ws);
  a.seg_slots = sm;
  a.seg_mats = reinterpret_cast<float*>(static_cast<char*>(ws) + segplan_plan_bytes(a.N, a.H, sm));
  a.qt = a.seg_mats + (size_t)3 * sm * a.H * kDK * kDK;
  a.seg_len = 0;
  a.nseg = 1;
  a.split_all = 0;
  // a 256-thread planner when the sequences and the slot capacity fit it (fewer wavefronts
  // at every barrier), else the 1024-thread one
  const int xc_max = segplan_long(a.T) ? kMaxItemTokens / kC : 0;
  if (a.N <= 256 && sm <= 256)
    chunk_segplan_kernel<256><<<1, 256, 0, stream>>>(a.cu, a.N, a.H, a.T, a.cus, sm,
                                                     L.mats_ok ? 1 : 0, L.qt_rows,
                                                     segplan_xc_min(a.T), xc_max, a.plan);
  else
    chunk_segplan_kernel<kMaxPlanSeqs><<<1, kMaxPlanSeqs, 0, stream>>>(
        a.cu, a.N, a.H, a.T, a.cus, sm, L.mats_ok ? 1 : 0, L.qt_rows, segplan_xc_min(a.T),
        xc_max, a.plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(2 * (size_t)a.H * sm);  // the largest plan
  const dim3 block(64 * (kPrepWaves + 4));
  if (a.erase) {  // Gated Delta Rule-2 gates
    if (per_channel) chunk_mfma_kernel<4, 2, true, true, kModeSeg><<<grid, block, 0, stream>>>(a);
    else chunk_mfma_kernel<4, 2, false, true, kModeSeg><<<grid, block, 0, stream>>>(a);
  } else {
    if (per_channel) chunk_mfma_kernel<4, 2, true, false, kModeSeg><<<grid, block, 0, stream>>>(a);
    else chunk_mfma_kernel<4, 2, false, false, kModeSeg><<<grid, block, 0, stream>>>(a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  seg_chain_kernel<<<dim3((unsigned)(a.N * a.H), kDK / 16), 512, 0, stream>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  seg_correct_kernel<<<dim3(1024), 256, 0, stream>>>(a);
  return hipGetLastError();
}

// Work list of the backward's two chain passes, which run at the same time: whole chains,
// longest first (splitting value columns adds work that the other pass could have used;
// measured 3% slower on H32 T65536 with halves).
hipError_t launch_chunk_plan(const ChunkArgs& a, hipStream_t stream) {
  if (!a.plan || !a.cu) return hipSuccess;  // equal-length batches need no work list
  chunk_plan_kernel<<<1, kMaxPlanSeqs, 0, stream>>>(a.cu, a.N, a.H, a.T, a.cus, 0, a.plan);
  return hipGetLastError();
}

hipError_t launch_chunk_mfma_hist(const ChunkArgs& args, bool per_channel, hipStream_t stream,
                                  bool build_plan) {
  ChunkArgs a = args;
  if (!a.hist || !chunk_mfma_supports(a.dk, a.dv, a.T)) return hipErrorInvalidValue;
  a.o = nullptr;
  a.seg_len = 0;
  return launch_mode<kModeHist>(a, per_channel, a.dv, stream, build_plan);
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
  // Gated Delta Rule-2 at dv = dk takes the segment plan instead (no kModePair variant)
  if (!chunk_mfma_supports(a.dk, a.dv, a.T) || (a.erase && a.dv == kDK))
    return hipErrorInvalidValue;
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
