/*
 * Float64 CPU oracle for gated linear attention with a per-key-channel
 * (diagonal) decay.  TEST INFRASTRUCTURE: only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load this file's library.  It
 * shares no code with the GPU path.
 *
 * What it computes (tokens t = 0..T-1, one (batch, head) sequence):
 *   state S_t in R^{dk x dv}, S_{-1} = h0 (zero unless given)
 *   S_t = diag(alpha_t) S_{t-1} + k_t v_t^T,   alpha_t = exp(g_t)  (g = log-gate)
 *   o_t = S_t^T q_t   (the token's own k_t v_t^T is included; its own gate is not
 *                      applied to it)
 * This is the fixed-size-state recurrence that the ZeCO pages build on:
 * "diagonal-decay gated linear attention" (atlas.scime.ai summary, section
 * "Limitations") with a state S in R^{dk x dv} (pith.science review, "Core
 * claim"); the decay acts per d_k row of S, which is why the All-Scan update
 * (pith.science review, "What carries the argument") scales whole rows.
 *
 * Backward, for the loss L = sum_t <do_t, o_t> + <dhT, S_{T-1}>:
 *   U_t = dL/dS_t:  U_{T-1} = dhT + q_{T-1} do_{T-1}^T,
 *                   U_t = diag(alpha_{t+1}) U_{t+1} + q_t do_t^T
 *   dq_t = S_t do_t,  dk_t = U_t v_t,  dv_t = U_t^T k_t,  dh0 = diag(alpha_0) U_0
 *   dg_{t,c} = alpha_{t,c} * sum_j S_{t-1}[c][j] U_t[c][j]          (direct form)
 *           = sum_{t'>=t} (q_{t'} dq_{t'} - k_{t'} dk_{t'})_c
 *             + sum_j S_{T-1}[c][j] dhT[c][j]                        (closed form)
 * The closed form follows from o depending on g only through q*exp(B) and
 * k*exp(-B) with B_t the running sum of g; the oracle's test suite checks it
 * against the direct form and against finite differences.
 *
 * Layouts (all row-major, contiguous): q, k, g, dq, dk, dg: [BH][T][dk];
 * v, o, do, dv: [BH][T][dv]; states h0, hT, dhT, dh0: [BH][dk][dv].
 *
 * Parallelism: the (batch*head) sequences are independent, and so are the
 * columns of S in the forward (o_t[j] needs only column j of S) and the rows
 * of S in the dq/dk sweeps.  The loops below only hand those independent
 * pieces to different threads; every element is accumulated in the same order
 * as in a single plain loop, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Forward recurrence.  hT may be NULL. */
void oracle_gla_fwd(int BH, int T, int dk, int dv,
                    const double* q, const double* k, const double* v, const double* g,
                    const double* h0, double* o, double* hT, int nthreads) {
  set_threads(nthreads);
  const long n_units = (long)BH * dv; /* one unit = one column j of one sequence */
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)dk); /* column j of S */
#pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < n_units; ++u) {
      const long bh = u / dv;
      const int j = (int)(u % dv);
      const double* qb = q + bh * (long)T * dk;
      const double* kb = k + bh * (long)T * dk;
      const double* vb = v + bh * (long)T * dv;
      const double* gb = g + bh * (long)T * dk;
      double* ob = o + bh * (long)T * dv;
      for (int c = 0; c < dk; ++c) S[c] = h0 ? h0[bh * (long)dk * dv + (long)c * dv + j] : 0.0;
      for (int t = 0; t < T; ++t) {
        const double vtj = vb[(long)t * dv + j];
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) {
          S[c] = exp(gb[(long)t * dk + c]) * S[c] + kb[(long)t * dk + c] * vtj;
          acc += qb[(long)t * dk + c] * S[c];
        }
        ob[(long)t * dv + j] = acc;
      }
      if (hT)
        for (int c = 0; c < dk; ++c) hT[bh * (long)dk * dv + (long)c * dv + j] = S[c];
    }
    free(S);
  }
}

/* Backward.  h0, dhT may be NULL (zero); dh0 may be NULL.
 * Three sweeps: rows of S forward (dq, and S_{T-1} for the dg constant),
 * rows of U in reverse (dk, dh0), columns of U in reverse (dv); then dg by
 * the closed form. */
void oracle_gla_bwd(int BH, int T, int dk, int dv,
                    const double* q, const double* k, const double* v, const double* g,
                    const double* dout, const double* h0, const double* dhT,
                    double* dq, double* dkk, double* dvv, double* dg, double* dh0,
                    int nthreads) {
  set_threads(nthreads);
  const long n_rows = (long)BH * dk;
  const long n_cols = (long)BH * dv;
  double* dg_const = (double*)calloc((size_t)n_rows, sizeof(double)); /* rowsum(S_{T-1} * dhT) */

  /* Sweep 1: rows of S, forward in t.  dq_t[c] = sum_j S_t[c][j] do_t[j]. */
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < n_rows; ++u) {
      const long bh = u / dk;
      const int c = (int)(u % dk);
      const double* kb = k + bh * (long)T * dk;
      const double* vb = v + bh * (long)T * dv;
      const double* gb = g + bh * (long)T * dk;
      const double* db = dout + bh * (long)T * dv;
      for (int j = 0; j < dv; ++j) S[j] = h0 ? h0[bh * (long)dk * dv + (long)c * dv + j] : 0.0;
      for (int t = 0; t < T; ++t) {
        const double a = exp(gb[(long)t * dk + c]);
        const double ktc = kb[(long)t * dk + c];
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
          S[j] = a * S[j] + ktc * vb[(long)t * dv + j];
          acc += S[j] * db[(long)t * dv + j];
        }
        dq[bh * (long)T * dk + (long)t * dk + c] = acc;
      }
      if (dhT) {
        double s = 0.0;
        for (int j = 0; j < dv; ++j) s += S[j] * dhT[bh * (long)dk * dv + (long)c * dv + j];
        dg_const[u] = s;
      }
    }
    free(S);
  }

  /* Sweep 2: rows of U, reverse in t.  dk_t[c] = sum_j U_t[c][j] v_t[j]. */
#pragma omp parallel
  {
    double* U = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < n_rows; ++u) {
      const long bh = u / dk;
      const int c = (int)(u % dk);
      const double* qb = q + bh * (long)T * dk;
      const double* vb = v + bh * (long)T * dv;
      const double* gb = g + bh * (long)T * dk;
      const double* db = dout + bh * (long)T * dv;
      for (int j = 0; j < dv; ++j) U[j] = dhT ? dhT[bh * (long)dk * dv + (long)c * dv + j] : 0.0;
      for (int t = T - 1; t >= 0; --t) {
        /* U now holds dL/dS_t minus the q_t do_t^T term: add it, then read out. */
        const double qtc = qb[(long)t * dk + c];
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
          U[j] += qtc * db[(long)t * dv + j];
          acc += U[j] * vb[(long)t * dv + j];
        }
        dkk[bh * (long)T * dk + (long)t * dk + c] = acc;
        /* carry to t-1: dL/dS_{t-1} gets diag(alpha_t) U_t */
        const double a = exp(gb[(long)t * dk + c]);
        for (int j = 0; j < dv; ++j) U[j] *= a;
      }
      if (dh0)
        for (int j = 0; j < dv; ++j) dh0[bh * (long)dk * dv + (long)c * dv + j] = U[j];
    }
    free(U);
  }

  /* Sweep 3: columns of U, reverse in t.  dv_t[j] = sum_c U_t[c][j] k_t[c]. */
#pragma omp parallel
  {
    double* U = (double*)malloc(sizeof(double) * (size_t)dk);
#pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < n_cols; ++u) {
      const long bh = u / dv;
      const int j = (int)(u % dv);
      const double* qb = q + bh * (long)T * dk;
      const double* kb = k + bh * (long)T * dk;
      const double* gb = g + bh * (long)T * dk;
      const double* db = dout + bh * (long)T * dv;
      for (int c = 0; c < dk; ++c) U[c] = dhT ? dhT[bh * (long)dk * dv + (long)c * dv + j] : 0.0;
      for (int t = T - 1; t >= 0; --t) {
        const double dtj = db[(long)t * dv + j];
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) {
          U[c] += qb[(long)t * dk + c] * dtj;
          acc += U[c] * kb[(long)t * dk + c];
        }
        dvv[bh * (long)T * dv + (long)t * dv + j] = acc;
        for (int c = 0; c < dk; ++c) U[c] *= exp(gb[(long)t * dk + c]);
      }
    }
    free(U);
  }

  /* dg, closed form: reverse running sum of q*dq - k*dk, plus rowsum(S_{T-1} * dhT). */
#pragma omp parallel for schedule(static)
  for (long u = 0; u < n_rows; ++u) {
    const long bh = u / dk;
    const int c = (int)(u % dk);
    double run = dg_const[u];
    for (int t = T - 1; t >= 0; --t) {
      const long i = bh * (long)T * dk + (long)t * dk + c;
      run += q[i] * dq[i] - k[i] * dkk[i];
      dg[i] = run;
    }
  }
  free(dg_const);
}

/* dg by its direct form, alpha_{t,c} * <S_{t-1}[c,:], U_t[c,:]>.  Keeps the
 * whole forward history of one row of S, so it is meant for small T. */
int oracle_gla_dg_direct(int BH, int T, int dk, int dv,
                         const double* q, const double* k, const double* v, const double* g,
                         const double* dout, const double* h0, const double* dhT,
                         double* dg, int nthreads) {
  set_threads(nthreads);
  const long n_rows = (long)BH * dk;
  int failed = 0;
#pragma omp parallel
  {
    double* hist = (double*)malloc(sizeof(double) * (size_t)(T + 1) * dv); /* S_{t-1} rows, t=0..T */
    double* U = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!hist || !U) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < n_rows; ++u) {
      if (!hist || !U) continue;
      const long bh = u / dk;
      const int c = (int)(u % dk);
      const double* qb = q + bh * (long)T * dk;
      const double* kb = k + bh * (long)T * dk;
      const double* vb = v + bh * (long)T * dv;
      const double* gb = g + bh * (long)T * dk;
      const double* db = dout + bh * (long)T * dv;
      /* hist[t] = S_{t-1}[c,:] */
      for (int j = 0; j < dv; ++j) hist[j] = h0 ? h0[bh * (long)dk * dv + (long)c * dv + j] : 0.0;
      for (int t = 0; t < T; ++t) {
        const double a = exp(gb[(long)t * dk + c]);
        for (int j = 0; j < dv; ++j)
          hist[(long)(t + 1) * dv + j] = a * hist[(long)t * dv + j] + kb[(long)t * dk + c] * vb[(long)t * dv + j];
      }
      for (int j = 0; j < dv; ++j) U[j] = dhT ? dhT[bh * (long)dk * dv + (long)c * dv + j] : 0.0;
      for (int t = T - 1; t >= 0; --t) {
        const double qtc = qb[(long)t * dk + c];
        for (int j = 0; j < dv; ++j) U[j] += qtc * db[(long)t * dv + j];
        const double a = exp(gb[(long)t * dk + c]);
        double s = 0.0;
        for (int j = 0; j < dv; ++j) s += hist[(long)t * dv + j] * U[j];
        dg[bh * (long)T * dk + (long)t * dk + c] = a * s;
        for (int j = 0; j < dv; ++j) U[j] *= a;
      }
    }
    free(hist);
    free(U);
  }
  return failed ? -1 : 0;
}
