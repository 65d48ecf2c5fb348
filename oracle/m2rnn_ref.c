/*
 * fp64 CPU oracle for the M²RNN matrix-state nonlinear recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg
 * load this library; the GPU product path never calls it and shares no code with it.
 *
 * Source: the reading notes "M²RNN：矩阵状态非线性 RNN 的容量、表达力与系统代价" on
 * arXiv:2603.14360v2 (cited below as "M²RNN notes").
 *   - forward:  §2.1, Eq. (10)-(12)   Z_t = tanh(H_{t-1} W + k_t v_t^T)
 *                                     H_t = f_t H_{t-1} + (1 - f_t) Z_t
 *                                     y_t = H_t^T q_t + w_r (.) v_t,      H_0 = 0 (or given)
 *   - backward: §2.7, the chain-rule BPTT written there in place of the paper's Algorithm 2:
 *               R_t = C_t + q_t u_t^T,  D_t = ((1-f_t) R_t) (.) (1 - Z_t (.) Z_t),
 *               C_{t-1} = f_t R_t + D_t W^T,  dL/df_t = <R_t, H_{t-1} - Z_t>_F,
 *               dL/dW = sum_t H_{t-1}^T D_t,  dL/dk_t = D_t v_t,  dL/dv_t = D_t^T k_t (+ w_r (.) u_t),
 *               dL/dq_t = H_t u_t,  and dL/dw_r = sum_t u_t (.) v_t for the value residual.
 *
 * Everything is plain fp64 in the order the equations are written: the contraction is a
 * straight loop over l ascending, tanh is the C library's, and no blocking or reordering is
 * applied.  Work is split over independent (batch, head) units only (one pthread per unit
 * stride), which does not change any unit's arithmetic.
 *
 * Layouts (row-major): q,k [B,T,N,K]; v,y,dy [B,T,N,V]; f [B,T,N]; W [N,V,V] with
 * (H W)[i][j] = sum_l H[i][l] W[l][j]; w_r [N,V]; H0,H_T,dH_T,dH0 [B,N,K,V].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t B, T, N, K, V;
  const double *q, *k, *v, *f, *W, *w_r, *H0, *dy, *dH_T;
  double *y, *H_T;
  double *dq, *dk, *dv, *df, *dW_unit, *dw_r_unit, *dH0;
  double clip; /* > 0: bound on every element of the gradient a step sends back to its input state */
  int64_t unit0, ustride;
  int status;
} job_t;

#define IDX_QK(b, t, n, i) ((((b) * J->T + (t)) * J->N + (n)) * J->K + (i))
#define IDX_V(b, t, n, j) ((((b) * J->T + (t)) * J->N + (n)) * J->V + (j))
#define IDX_F(b, t, n) (((b) * J->T + (t)) * J->N + (n))
#define IDX_S(b, n, i, j) ((((b) * J->N + (n)) * J->K + (i)) * J->V + (j))

/* One step of Eq. (10)-(11): Hnext from Hprev (both K x V).  P is K x V scratch. */
static void step_state(const job_t* J, int64_t b, int64_t t, int64_t n, const double* Hprev,
                       double* Hnext, double* Z, double* P) {
  const int64_t K = J->K, V = J->V;
  const double* W = J->W + n * V * V;
  const double ft = J->f[IDX_F(b, t, n)];
  for (int64_t i = 0; i < K; ++i) {
    const double ki = J->k[IDX_QK(b, t, n, i)];
    for (int64_t j = 0; j < V; ++j) {
      double s = 0.0;
      for (int64_t l = 0; l < V; ++l) s += Hprev[i * V + l] * W[l * V + j];
      P[i * V + j] = s + ki * J->v[IDX_V(b, t, n, j)];
    }
  }
  for (int64_t e = 0; e < K * V; ++e) {
    Z[e] = tanh(P[e]);
    Hnext[e] = ft * Hprev[e] + (1.0 - ft) * Z[e];
  }
}

static void* fwd_worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int64_t K = J->K, V = J->V;
  double* buf = (double*)malloc(sizeof(double) * 4 * (size_t)(K * V));
  if (!buf) { J->status = -1; return NULL; }
  double *H = buf, *Hn = buf + K * V, *Z = buf + 2 * K * V, *P = buf + 3 * K * V;
  for (int64_t u = J->unit0; u < J->B * J->N; u += J->ustride) {
    const int64_t b = u / J->N, n = u % J->N;
    for (int64_t e = 0; e < K * V; ++e) H[e] = J->H0 ? J->H0[IDX_S(b, n, 0, 0) + e] : 0.0;
    for (int64_t t = 0; t < J->T; ++t) {
      step_state(J, b, t, n, H, Hn, Z, P);
      double* tmp = H; H = Hn; Hn = tmp;
      /* Eq. (12): readout from the post-update state. */
      for (int64_t j = 0; j < V; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < K; ++i) s += H[i * V + j] * J->q[IDX_QK(b, t, n, i)];
        J->y[IDX_V(b, t, n, j)] = s + J->w_r[n * V + j] * J->v[IDX_V(b, t, n, j)];
      }
    }
    if (J->H_T)
      for (int64_t e = 0; e < K * V; ++e) J->H_T[IDX_S(b, n, 0, 0) + e] = H[e];
  }
  free(buf);
  return NULL;
}

static void* bwd_worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int64_t K = J->K, V = J->V, T = J->T;
  const size_t kv = (size_t)(K * V);
  /* All states H_0..H_T of one unit, plus scratch. */
  double* Hs = (double*)malloc(sizeof(double) * kv * (size_t)(T + 1));
  double* buf = (double*)malloc(sizeof(double) * kv * 5);
  if (!Hs || !buf) { free(Hs); free(buf); J->status = -1; return NULL; }
  double *Z = buf, *P = buf + kv, *C = buf + 2 * kv, *R = buf + 3 * kv, *D = buf + 4 * kv;
  for (int64_t u = J->unit0; u < J->B * J->N; u += J->ustride) {
    const int64_t b = u / J->N, n = u % J->N;
    const double* W = J->W + n * V * V;
    double* dWu = J->dW_unit + (size_t)u * V * V;
    double* dwru = J->dw_r_unit + (size_t)u * V;
    for (size_t e = 0; e < kv; ++e) Hs[e] = J->H0 ? J->H0[IDX_S(b, n, 0, 0) + e] : 0.0;
    for (int64_t t = 0; t < T; ++t) step_state(J, b, t, n, Hs + kv * t, Hs + kv * (t + 1), Z, P);
    for (size_t e = 0; e < kv; ++e) C[e] = J->dH_T ? J->dH_T[IDX_S(b, n, 0, 0) + e] : 0.0;
    memset(dWu, 0, sizeof(double) * V * V);
    memset(dwru, 0, sizeof(double) * V);
    for (int64_t t = T - 1; t >= 0; --t) {
      const double* Hprev = Hs + kv * t;
      const double* Hcur = Hs + kv * (t + 1);
      const double ft = J->f[IDX_F(b, t, n)];
      const double* ut = J->dy + IDX_V(b, t, n, 0);
      const double* qt = J->q + IDX_QK(b, t, n, 0);
      const double* kt = J->k + IDX_QK(b, t, n, 0);
      const double* vt = J->v + IDX_V(b, t, n, 0);
      /* Recompute Z_t from H_{t-1} (Eq. 10). */
      for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < V; ++j) {
          double s = 0.0;
          for (int64_t l = 0; l < V; ++l) s += Hprev[i * V + l] * W[l * V + j];
          Z[i * V + j] = tanh(s + kt[i] * vt[j]);
        }
      /* R_t = C_t + q_t u_t^T;  D_t = ((1 - f_t) R_t) (.) (1 - Z_t (.) Z_t). */
      double dft = 0.0;
      for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < V; ++j) {
          const int64_t e = i * V + j;
          R[e] = C[e] + qt[i] * ut[j];
          D[e] = ((1.0 - ft) * R[e]) * (1.0 - Z[e] * Z[e]);
          dft += R[e] * (Hprev[e] - Z[e]);
        }
      J->df[IDX_F(b, t, n)] = dft;
      for (int64_t i = 0; i < K; ++i) {
        double sq = 0.0, sk = 0.0;
        for (int64_t j = 0; j < V; ++j) {
          sq += Hcur[i * V + j] * ut[j];
          sk += D[i * V + j] * vt[j];
        }
        J->dq[IDX_QK(b, t, n, i)] = sq;
        J->dk[IDX_QK(b, t, n, i)] = sk;
      }
      for (int64_t j = 0; j < V; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < K; ++i) s += D[i * V + j] * kt[i];
        J->dv[IDX_V(b, t, n, j)] = s + J->w_r[n * V + j] * ut[j];
        dwru[j] += ut[j] * vt[j];
      }
      for (int64_t l = 0; l < V; ++l)
        for (int64_t j = 0; j < V; ++j) {
          double s = 0.0;
          for (int64_t i = 0; i < K; ++i) s += Hprev[i * V + l] * D[i * V + j];
          dWu[l * V + j] += s;
        }
      /* C_{t-1} = f_t R_t + D_t W^T, the gradient step t sends back to H_{t-1}; with clipping
         (the notes' §2.3: the recurrent-state gradient is clipped at every BPTT step), each element
         is clamped to [-clip, clip] before it is used. */
      for (int64_t i = 0; i < K; ++i)
        for (int64_t l = 0; l < V; ++l) {
          double s = 0.0;
          for (int64_t j = 0; j < V; ++j) s += D[i * V + j] * W[l * V + j];
          double c = ft * R[i * V + l] + s;
          if (J->clip > 0.0) c = c > J->clip ? J->clip : (c < -J->clip ? -J->clip : c);
          C[i * V + l] = c;
        }
    }
    if (J->dH0)
      for (size_t e = 0; e < kv; ++e) J->dH0[IDX_S(b, n, 0, 0) + e] = C[e];
  }
  free(Hs);
  free(buf);
  return NULL;
}

static int run_jobs(job_t* proto, int nthreads, void* (*fn)(void*)) {
  const int64_t units = proto->B * proto->N;
  if (units == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > units) nthreads = (int)units;
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return -1; }
  int rc = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = *proto;
    jobs[i].unit0 = i;
    jobs[i].ustride = nthreads;
    jobs[i].status = 0;
  }
  for (int i = 1; i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, fn, &jobs[i]) != 0) { jobs[i].status = -1; th[i] = 0; fn(&jobs[i]); jobs[i].status = 0; }
  fn(&jobs[0]);
  for (int i = 1; i < nthreads; ++i)
    if (th[i]) pthread_join(th[i], NULL);
  for (int i = 0; i < nthreads; ++i) rc |= jobs[i].status;
  free(jobs);
  free(th);
  return rc;
}

/* Forward, Eq. (10)-(12).  H0 and H_T may be NULL (H0 = 0; H_T not written).  Returns 0 on
 * success, -1 on allocation failure, -2 on bad sizes. */
int m2rnn_ref_fwd(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V, const double* q, const double* k,
                  const double* v, const double* f, const double* W, const double* w_r, const double* H0,
                  double* y, double* H_T, int nthreads) {
  if (B < 0 || T < 0 || N < 0 || K <= 0 || V <= 0) return -2;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.T = T; J.N = N; J.K = K; J.V = V;
  J.q = q; J.k = k; J.v = v; J.f = f; J.W = W; J.w_r = w_r; J.H0 = H0;
  J.y = y; J.H_T = H_T;
  return run_jobs(&J, nthreads, fwd_worker);
}

/* Backward (BPTT of §2.7) for L = sum_t <dy_t, y_t> + <dH_T, H_T>.  dH_T and H0 may be NULL
 * (zeros); dH0 may be NULL.  dW [N,V,V] and dw_r [N,V] are summed over batch (b ascending). */
int m2rnn_ref_bwd(int64_t B, int64_t T, int64_t N, int64_t K, int64_t V, const double* q, const double* k,
                  const double* v, const double* f, const double* W, const double* w_r, const double* H0,
                  const double* dy, const double* dH_T, double clip, double* dq, double* dk, double* dv,
                  double* df, double* dW, double* dw_r, double* dH0, int nthreads) {
  if (B < 0 || T < 0 || N < 0 || K <= 0 || V <= 0) return -2;
  double* dWu = (double*)calloc((size_t)(B * N * V * V) + 1, sizeof(double));
  double* dwru = (double*)calloc((size_t)(B * N * V) + 1, sizeof(double));
  if (!dWu || !dwru) { free(dWu); free(dwru); return -1; }
  job_t J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.T = T; J.N = N; J.K = K; J.V = V;
  J.q = q; J.k = k; J.v = v; J.f = f; J.W = W; J.w_r = w_r; J.H0 = H0; J.dy = dy; J.dH_T = dH_T;
  J.clip = clip;
  J.dq = dq; J.dk = dk; J.dv = dv; J.df = df; J.dW_unit = dWu; J.dw_r_unit = dwru; J.dH0 = dH0;
  int rc = run_jobs(&J, nthreads, bwd_worker);
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t e = 0; e < V * V; ++e) {
      double s = 0.0;
      for (int64_t b = 0; b < B; ++b) s += dWu[(b * N + n) * V * V + e];
      dW[n * V * V + e] = s;
    }
    for (int64_t j = 0; j < V; ++j) {
      double s = 0.0;
      for (int64_t b = 0; b < B; ++b) s += dwru[(b * N + n) * V + j];
      dw_r[n * V + j] = s;
    }
  }
  free(dWu);
  free(dwru);
  return rc;
}
