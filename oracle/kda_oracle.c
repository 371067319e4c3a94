/*
 * fp64 CPU oracle for the gated delta rule with per-key-channel decay
 * (Kimi Delta Attention, "KDA"); Gated DeltaNet is the case of one decay per head.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline call this file. It shares no code, header or constant with the HIP
 * library, and the HIP library never calls it.
 *
 * What it computes (one independent chain = one sequence of one head):
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
 *   S in R^{dk x dv} (rows = key channels), alpha_t = exp(g_t).
 * Source: "Token Mixer I", section "Kimi Delta Attention: Improving Delta Rule with
 * Fine-grained Gating", boxed recurrence. The order of operations per token is the
 * decay-then-delta form of the page "KDA 与 Gated DeltaNet：线性注意力怎样读写有限状态",
 * section 2 (S~ = Diag(alpha) S, then S = S~ + beta k (v - S~^T k)^T), which is also
 * the five-line pseudo-code of its section 4:
 *   1. a = exp(g_t)            (g_t broadcast over the key channels for one decay per head)
 *   2. S <- Diag(a) S          (row i, the key channel, scaled by a[i])
 *   3. p = S^T k_t             (the prediction of the value from the decayed state)
 *   4. S <- S + k_t (w v_t - e p)^T
 *   5. o_t = S^T q_t
 * With e = w = beta_t this is the method. Other scalar (e, w) exist for the pins of the
 * tests (e = 0, w = 1 and alpha = 1 give plain linear attention).
 *
 * Gated Delta Rule-2 ("Token Mixer I", section "Gated DeltaNet-2: Decoupling Erase and
 * Write", the residual of its fast-weight section) replaces the scalar gate by a
 * per-key-channel erase gate b_t in [0,1]^dk and a per-value-channel write gate
 * w_t in [0,1]^dv: with S~ = Diag(alpha) S,
 *   S_t = S~ + k_t (w_t * v_t - S~^T (b_t * k_t))^T      (* elementwise)
 * so steps 3-4 read p = S~^T (b_t * k_t) and write k_t (w_t * v_t - p)^T. b = beta 1 and
 * w = beta 1 give the method again.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* One chain. Row r of the chain is row (off + r) of every per-token array. */
static void oracle_chain(int dk, int dv, int64_t off, int64_t len,
                         const double* q, const double* k, const double* v,
                         const double* g, int gate_per_channel, const double* beta,
                         const double* erase, const double* write,
                         const double* erase_vec, const double* write_vec,
                         const double* s0, double* o, double* s_final,
                         double* S, double* a, double* p, double* d, double* ek) {
  if (s0)
    memcpy(S, s0, sizeof(double) * (size_t)dk * dv);
  else
    memset(S, 0, sizeof(double) * (size_t)dk * dv);

  for (int64_t t = 0; t < len; ++t) {
    const int64_t row = off + t;
    const double* qt = q + row * dk;
    const double* kt = k + row * dk;
    const double* vt = v + row * dv;
    const double bt = beta[row];
    const double et = erase ? erase[row] : bt;
    const double wt = write ? write[row] : bt;

    /* 1-2: decay each key-channel row of the state */
    for (int i = 0; i < dk; ++i)
      a[i] = exp(gate_per_channel ? g[row * dk + i] : g[row]);
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a[i];

    /* 3: prediction p = S^T (e k), e the erase gate of each key channel */
    for (int i = 0; i < dk; ++i) ek[i] = (erase_vec ? erase_vec[row * dk + i] : et) * kt[i];
    for (int j = 0; j < dv; ++j) p[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) p[j] += S[(size_t)i * dv + j] * ek[i];

    /* 4: rank-one correction along k, w the write gate of each value channel */
    for (int j = 0; j < dv; ++j) d[j] = (write_vec ? write_vec[row * dv + j] : wt) * vt[j] - p[j];
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * d[j];

    /* 5: read-out o = S^T q */
    double* ot = o + row * dv;
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * qt[i];
  }
  if (s_final) memcpy(s_final, S, sizeof(double) * (size_t)dk * dv);
}

/*
 * Runs n_chains independent chains, in parallel over chains (OpenMP).
 *   row_off[c], row_len[c] : first row and number of tokens of chain c
 *   q, k : [rows, dk]   v, o : [rows, dv]   g : [rows, dk] or [rows]   beta : [rows]
 *   erase, write : [rows] or NULL (NULL = beta, the method itself)
 *   erase_vec    : [rows, dk] or NULL; write_vec : [rows, dv] or NULL (Gated Delta Rule-2
 *                  gates; when given they replace erase / write)
 *   s0, s_final  : [n_chains, dk, dv] or NULL (s0 NULL = zero initial state)
 *   n_threads    : OpenMP threads (<= 0: the runtime default)
 * Returns 0, or -1 if a work buffer could not be allocated.
 */
int oracle_kda_chains(int n_chains, int dk, int dv,
                      const int64_t* row_off, const int64_t* row_len,
                      const double* q, const double* k, const double* v,
                      const double* g, int gate_per_channel, const double* beta,
                      const double* erase, const double* write,
                      const double* erase_vec, const double* write_vec,
                      const double* s0, double* o, double* s_final, int n_threads) {
  int failed = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel num_threads(n_threads) reduction(| : failed)
#endif
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* p = (double*)malloc(sizeof(double) * (size_t)dv);
    double* d = (double*)malloc(sizeof(double) * (size_t)dv);
    double* ek = (double*)malloc(sizeof(double) * (size_t)dk);
    const int have_buffers = S && a && p && d && ek;
    if (!have_buffers) failed = 1;
    /* every thread reaches the work-sharing loop; one without buffers computes nothing */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int c = 0; c < n_chains; ++c) {
      if (!have_buffers) continue;
      oracle_chain(dk, dv, row_off[c], row_len[c], q, k, v, g, gate_per_channel, beta,
                   erase, write, erase_vec, write_vec, s0 ? s0 + (size_t)c * dk * dv : NULL, o,
                   s_final ? s_final + (size_t)c * dk * dv : NULL, S, a, p, d, ek);
    }
    free(S);
    free(a);
    free(p);
    free(d);
    free(ek);
  }
  return failed ? -1 : 0;
}
