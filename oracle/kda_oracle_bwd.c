/*
 * fp64 CPU oracle for the backward pass of the gated delta rule (KDA, Gated DeltaNet,
 * Gated Delta Rule-2): the gradients of a scalar loss with respect to every input of
 * the forward recurrence of kda_oracle.c, given the loss's gradients with respect to
 * the outputs o_t and the final state S_T.
 *
 * TEST INFRASTRUCTURE, like kda_oracle.c: only the tests use it; it shares nothing with
 * the HIP library.
 *
 * The forward step of a token ("Token Mixer I", section "Kimi Delta Attention", boxed
 * recurrence, in the decay-then-delta order of the page "KDA 与 Gated DeltaNet：线性注意力
 * 怎样读写有限状态", section 2; the erase / write gates of section "Gated DeltaNet-2"):
 *   S~ = Diag(a) S,  a = exp(g)        p = S~^T (e * k)        d = w * v - p
 *   S' = S~ + k d^T                    o = S'^T q
 * with e = w = beta (scalars) for KDA / Gated DeltaNet, or the vectors e [dk], w [dv].
 * The backward pass needs only the chain rule, applied to these five lines in reverse
 * order (the pages give no backward equations; their chunkwise section says the
 * backward has the forward's shapes). With dS' the gradient reaching S' (from later
 * tokens, or from S_T), per token in reverse:
 *   dS' += q do^T            dq = S' do
 *   dd   = dS'^T k           dk = dS' d
 *   dw   = dd * v            dv = dd * w
 *   dp   = -dd
 *   dS~  = dS' + (e * k) dp^T
 *   r    = S~ dp             dk += e * r        de = k * r
 *   dg_i = sum_j dS~_ij S~_ij   (per key channel; summed over i for one decay per head)
 *   dS   = Diag(a) dS~       (the gradient reaching the previous state)
 * For KDA, e and w are the same beta: dbeta = sum_i de_i + sum_j dw_j.
 *
 * Memory: the forward states are recomputed segment by segment from checkpoints taken
 * every SEG tokens, so a chain of length L holds ceil(L / SEG) + SEG states.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SEG 64

typedef struct {
  int dk, dv, per_channel;
  const double *q, *k, *v, *g, *beta, *e_vec, *w_vec;
} chain_in;

/* The decay of token row (a[i] = exp(g)). */
static void decay(const chain_in* c, int64_t row, double* a) {
  for (int i = 0; i < c->dk; ++i)
    a[i] = exp(c->per_channel ? c->g[row * c->dk + i] : c->g[row]);
}

/* Erase-gated key e * k of token row. */
static void gated_key(const chain_in* c, int64_t row, double* ek) {
  const double* kt = c->k + row * c->dk;
  for (int i = 0; i < c->dk; ++i)
    ek[i] = (c->e_vec ? c->e_vec[row * c->dk + i] : c->beta[row]) * kt[i];
}

/* One forward step S <- S' of token row. On return St holds S~ (decayed, before the
 * rank-one update) when St != NULL, and d the write residual. */
static void step(const chain_in* c, int64_t row, double* S, double* St, double* a, double* ek,
                 double* d) {
  const int dk = c->dk, dv = c->dv;
  const double* kt = c->k + row * dk;
  const double* vt = c->v + row * dv;
  decay(c, row, a);
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a[i];
  if (St) memcpy(St, S, sizeof(double) * (size_t)dk * dv);
  gated_key(c, row, ek);
  for (int j = 0; j < dv; ++j) {
    double p = 0.0;
    for (int i = 0; i < dk; ++i) p += S[(size_t)i * dv + j] * ek[i];
    d[j] = (c->w_vec ? c->w_vec[row * dv + j] : c->beta[row]) * vt[j] - p;
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * d[j];
}

typedef struct {
  double *ck, *Sseg, *dvec, *S, *dS, *a, *ek, *dd, *r;
} work;

static int work_alloc(work* w, int dk, int dv, int64_t max_len) {
  const size_t st = (size_t)dk * dv;
  const int64_t n_ck = (max_len + SEG - 1) / SEG + 1;
  w->ck = (double*)malloc(sizeof(double) * st * (size_t)n_ck);
  w->Sseg = (double*)malloc(sizeof(double) * st * SEG);
  w->dvec = (double*)malloc(sizeof(double) * (size_t)dv * SEG);
  w->S = (double*)malloc(sizeof(double) * st);
  w->dS = (double*)malloc(sizeof(double) * st);
  w->a = (double*)malloc(sizeof(double) * (size_t)dk);
  w->ek = (double*)malloc(sizeof(double) * (size_t)dk);
  w->dd = (double*)malloc(sizeof(double) * (size_t)dv);
  w->r = (double*)malloc(sizeof(double) * (size_t)dk);
  return w->ck && w->Sseg && w->dvec && w->S && w->dS && w->a && w->ek && w->dd && w->r;
}

static void work_free(work* w) {
  free(w->ck); free(w->Sseg); free(w->dvec); free(w->S); free(w->dS);
  free(w->a); free(w->ek); free(w->dd); free(w->r);
}

/* Gradients of one chain (rows off .. off + len - 1). */
static void chain_bwd(const chain_in* c, int64_t off, int64_t len, const double* s0,
                      const double* dout, const double* dsT, double* dq, double* dkk,
                      double* dvv, double* dg, double* dbeta, double* de_vec, double* dw_vec,
                      double* ds0, work* w) {
  const int dk = c->dk, dv = c->dv;
  const size_t st = (size_t)dk * dv;
  /* forward: checkpoint the state before every segment */
  if (s0) memcpy(w->S, s0, sizeof(double) * st);
  else memset(w->S, 0, sizeof(double) * st);
  const int64_t n_seg = (len + SEG - 1) / SEG;
  for (int64_t s = 0; s < n_seg; ++s) {
    memcpy(w->ck + (size_t)s * st, w->S, sizeof(double) * st);
    const int64_t t1 = (s + 1) * SEG < len ? (s + 1) * SEG : len;
    for (int64_t t = s * SEG; t < t1; ++t) step(c, off + t, w->S, NULL, w->a, w->ek, w->dd);
  }
  /* backward, segment by segment from the last */
  if (dsT) memcpy(w->dS, dsT, sizeof(double) * st);
  else memset(w->dS, 0, sizeof(double) * st);
  for (int64_t s = n_seg - 1; s >= 0; --s) {
    const int64_t t0 = s * SEG;
    const int64_t t1 = (s + 1) * SEG < len ? (s + 1) * SEG : len;
    /* recompute S~ and d of every token of the segment */
    memcpy(w->S, w->ck + (size_t)s * st, sizeof(double) * st);
    for (int64_t t = t0; t < t1; ++t)
      step(c, off + t, w->S, w->Sseg + (size_t)(t - t0) * st, w->a, w->ek,
           w->dvec + (size_t)(t - t0) * dv);
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const int64_t row = off + t;
      const double* St = w->Sseg + (size_t)(t - t0) * st;  /* S~ of this token */
      const double* d = w->dvec + (size_t)(t - t0) * dv;
      const double* qt = c->q + row * dk;
      const double* kt = c->k + row * dk;
      const double* vt = c->v + row * dv;
      const double* dot = dout + row * dv;
      /* S' = S~ + k d^T, rebuilt in S */
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
          w->S[(size_t)i * dv + j] = St[(size_t)i * dv + j] + kt[i] * d[j];
      /* o = S'^T q */
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
          w->dS[(size_t)i * dv + j] += qt[i] * dot[j];
          acc += w->S[(size_t)i * dv + j] * dot[j];
        }
        dq[row * dk + i] = acc;
      }
      /* S' = S~ + k d^T */
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += w->dS[(size_t)i * dv + j] * kt[i];
        w->dd[j] = acc;
      }
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += w->dS[(size_t)i * dv + j] * d[j];
        dkk[row * dk + i] = acc;
      }
      /* d = w * v - p */
      double dw_sum = 0.0;
      for (int j = 0; j < dv; ++j) {
        const double wj = c->w_vec ? c->w_vec[row * dv + j] : c->beta[row];
        dvv[row * dv + j] = w->dd[j] * wj;
        if (dw_vec) dw_vec[row * dv + j] = w->dd[j] * vt[j];
        dw_sum += w->dd[j] * vt[j];
      }
      /* p = S~^T (e k): dS~ = dS' + (e k) dp^T with dp = -dd, and r = S~ dp */
      gated_key(c, row, w->ek);
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
          w->dS[(size_t)i * dv + j] -= w->ek[i] * w->dd[j];
          acc -= St[(size_t)i * dv + j] * w->dd[j];
        }
        w->r[i] = acc;
      }
      double de_sum = 0.0;
      for (int i = 0; i < dk; ++i) {
        const double ei = c->e_vec ? c->e_vec[row * dk + i] : c->beta[row];
        dkk[row * dk + i] += ei * w->r[i];
        if (de_vec) de_vec[row * dk + i] = kt[i] * w->r[i];
        de_sum += kt[i] * w->r[i];
      }
      if (dbeta) dbeta[row] = de_sum + dw_sum;
      /* S~ = Diag(a) S: dg from dS~ and S~, then the gradient of the previous state */
      decay(c, row, w->a);
      double dg_sum = 0.0;
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
          acc += w->dS[(size_t)i * dv + j] * St[(size_t)i * dv + j];
          w->dS[(size_t)i * dv + j] *= w->a[i];
        }
        if (c->per_channel) dg[row * dk + i] = acc;
        dg_sum += acc;
      }
      if (!c->per_channel) dg[row] = dg_sum;
    }
  }
  if (ds0) memcpy(ds0, w->dS, sizeof(double) * st);
}

/*
 * Backward of oracle_kda_chains, in parallel over chains (OpenMP).
 *   row_off, row_len, q, k, v, g, gate_per_channel, beta, s0: as in oracle_kda_chains
 *   erase_vec [rows, dk], write_vec [rows, dv]: the Gated Delta Rule-2 gates, both NULL
 *                       for KDA / Gated DeltaNet (both gates are then beta)
 *   dout [rows, dv]     gradient of the loss with respect to o
 *   dsT [chains, dk, dv] gradient with respect to the final states, or NULL (zero)
 * Outputs (every row of every chain is written):
 *   dq, dk [rows, dk]; dv [rows, dv]; dg [rows, dk] or [rows] (like g);
 *   dbeta [rows] (KDA; may be NULL for Gated Delta Rule-2);
 *   derase [rows, dk], dwrite [rows, dv] (Gated Delta Rule-2; may be NULL);
 *   ds0 [chains, dk, dv] or NULL.
 * Returns 0, or -1 if a work buffer could not be allocated.
 */
int oracle_kda_chains_bwd(int n_chains, int dk, int dv, const int64_t* row_off,
                          const int64_t* row_len, const double* q, const double* k,
                          const double* v, const double* g, int gate_per_channel,
                          const double* beta, const double* erase_vec, const double* write_vec,
                          const double* s0, const double* dout, const double* dsT, double* dq,
                          double* dkk, double* dvv, double* dg, double* dbeta, double* derase,
                          double* dwrite, double* ds0, int n_threads) {
  chain_in c = {dk, dv, gate_per_channel, q, k, v, g, beta, erase_vec, write_vec};
  int64_t max_len = 1;
  for (int i = 0; i < n_chains; ++i)
    if (row_len[i] > max_len) max_len = row_len[i];
  int failed = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel num_threads(n_threads) reduction(| : failed)
#endif
  {
    work w;
    const int ok = work_alloc(&w, dk, dv, max_len);
    if (!ok) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int i = 0; i < n_chains; ++i) {
      if (!ok) continue;
      const size_t st = (size_t)dk * dv;
      chain_bwd(&c, row_off[i], row_len[i], s0 ? s0 + i * st : NULL, dout,
                dsT ? dsT + i * st : NULL, dq, dkk, dvv, dg, dbeta, derase, dwrite,
                ds0 ? ds0 + i * st : NULL, &w);
    }
    work_free(&w);
  }
  return failed ? -1 : 0;
}
