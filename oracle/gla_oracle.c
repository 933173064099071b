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

/* Forward recurrence.  hT may be NULL.  If hs is not NULL, the state after tokens
 * every-1, 2*every-1, ... is stored in hs [BH][T/every][dk][dv].  Work unit: one sequence and a
 * block of up to JB columns of S (columns never interact); exp(g) is taken once per (t, c) for
 * the block. */
#define JB 16
void oracle_gla_fwd(int BH, int T, int dk, int dv,
                    const double* q, const double* k, const double* v, const double* g,
                    const double* h0, double* o, double* hT, double* hs, int every, int nthreads) {
  set_threads(nthreads);
  const int nblk = (dv + JB - 1) / JB;
  const int nrec = (hs && every > 0) ? T / every : 0;
  const long n_units = (long)BH * nblk;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * JB); /* S[c][jj], columns j0.. */
#pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < n_units; ++u) {
      const long bh = u / nblk;
      const int j0 = (int)(u % nblk) * JB;
      const int nj = dv - j0 < JB ? dv - j0 : JB;
      const double* qb = q + bh * (long)T * dk;
      const double* kb = k + bh * (long)T * dk;
      const double* vb = v + bh * (long)T * dv;
      const double* gb = g + bh * (long)T * dk;
      double* ob = o + bh * (long)T * dv;
      for (int c = 0; c < dk; ++c)
        for (int jj = 0; jj < nj; ++jj)
          S[c * JB + jj] = h0 ? h0[bh * (long)dk * dv + (long)c * dv + j0 + jj] : 0.0;
      for (int t = 0; t < T; ++t) {
        double acc[JB];
        for (int jj = 0; jj < nj; ++jj) acc[jj] = 0.0;
        for (int c = 0; c < dk; ++c) {
          const double a = exp(gb[(long)t * dk + c]);
          const double ktc = kb[(long)t * dk + c];
          const double qtc = qb[(long)t * dk + c];
          for (int jj = 0; jj < nj; ++jj) {
            S[c * JB + jj] = a * S[c * JB + jj] + ktc * vb[(long)t * dv + j0 + jj];
            acc[jj] += qtc * S[c * JB + jj];
          }
        }
        for (int jj = 0; jj < nj; ++jj) ob[(long)t * dv + j0 + jj] = acc[jj];
        if (nrec && (t + 1) % every == 0) {
          double* hb = hs + (bh * (long)nrec + (t + 1) / every - 1) * dk * dv;
          for (int c = 0; c < dk; ++c)
            for (int jj = 0; jj < nj; ++jj) hb[(long)c * dv + j0 + jj] = S[c * JB + jj];
        }
      }
      if (hT)
        for (int c = 0; c < dk; ++c)
          for (int jj = 0; jj < nj; ++jj) hT[bh * (long)dk * dv + (long)c * dv + j0 + jj] = S[c * JB + jj];
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

  /* Sweep 3: columns of U, reverse in t, in blocks of up to JB columns.
   * dv_t[j] = sum_c U_t[c][j] k_t[c]. */
  {
    const int nblk = (dv + JB - 1) / JB;
    const long n_units = (long)BH * nblk;
#pragma omp parallel
    {
      double* U = (double*)malloc(sizeof(double) * (size_t)dk * JB);
#pragma omp for schedule(dynamic, 1)
      for (long u = 0; u < n_units; ++u) {
        const long bh = u / nblk;
        const int j0 = (int)(u % nblk) * JB;
        const int nj = dv - j0 < JB ? dv - j0 : JB;
        const double* qb = q + bh * (long)T * dk;
        const double* kb = k + bh * (long)T * dk;
        const double* gb = g + bh * (long)T * dk;
        const double* db = dout + bh * (long)T * dv;
        for (int c = 0; c < dk; ++c)
          for (int jj = 0; jj < nj; ++jj)
            U[c * JB + jj] = dhT ? dhT[bh * (long)dk * dv + (long)c * dv + j0 + jj] : 0.0;
        for (int t = T - 1; t >= 0; --t) {
          double acc[JB];
          for (int jj = 0; jj < nj; ++jj) acc[jj] = 0.0;
          for (int c = 0; c < dk; ++c) {
            const double qtc = qb[(long)t * dk + c];
            const double ktc = kb[(long)t * dk + c];
            for (int jj = 0; jj < nj; ++jj) {
              U[c * JB + jj] += qtc * db[(long)t * dv + j0 + jj];
              acc[jj] += U[c * JB + jj] * ktc;
            }
          }
          for (int jj = 0; jj < nj; ++jj) dvv[bh * (long)T * dv + (long)t * dv + j0 + jj] = acc[jj];
          for (int c = 0; c < dk; ++c) {
            const double a = exp(gb[(long)t * dk + c]);
            for (int jj = 0; jj < nj; ++jj) U[c * JB + jj] *= a;
          }
        }
      }
      free(U);
    }
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
