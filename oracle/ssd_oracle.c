/*
 * ssd_oracle.c -- fp64 CPU oracle for the Mamba-2 SSD forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load this file's
 * library; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do.  It shares no code, header or constant with the HIP library.
 *
 * Sources (web pages, cited by title):
 *   P1 = "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
 *         Tensor Cores with cuTile" (disconfirmai.com digest of the NVIDIA
 *         Developer Blog post on Mamba-2 forward kernels in cuTile).
 *
 * What is computed: the plain token-by-token recurrence, not the chunked
 * algorithm.  P1's opening paragraph describes Mamba-2 as a fixed-size hidden
 * state updated once per token; its jump-formula paragraph fixes the
 * decay-free update as an accumulation of outer products b x^T (state = N x P
 * per head, b stacked as rows of the N side) and says the decay enters as a
 * per-token multiplicative factor whose logarithms are summed.  The standard
 * Mamba-2 reading of that, used here, is, for batch b, head h, group
 * g = h / (H/G):
 *
 *     h_{-1} = h0[b,h]                     (zeros when no initial state)
 *     h_t    = exp(dt[b,t,h] * A[h]) * h_{t-1} + dt[b,t,h] * B[b,t,g,:] x[b,t,h,:]^T
 *     y_t    = C[b,t,g,:]^T h_t + D[h] * x[b,t,h,:]        (P1 compute_out
 *              paragraph: carried-state/interaction term plus skip connection)
 *     final  = h_{L-1}
 *
 * Every input is read as float and widened to double; all arithmetic is
 * double, no fast-math, no reassociation beyond the loops written here.
 *
 * Optional chunk bookkeeping (for checking the kernels' intermediates by
 * definition rather than by the chunked algorithm):
 *   reset_each_chunk = 0: boundary[c] = h_{cQ-1}, the state entering chunk c
 *                         (boundary[0] = h0).
 *   reset_each_chunk = 1: the state is zeroed at the start of every chunk and
 *                         boundary[c] = the state after the chunk's last token,
 *                         i.e. the chunk's own contribution from a zero start.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t Bsz, L, H, P, N, G;
  const float *x, *dt, *A, *Bm, *Cm, *D;
  const double* h0;
  int64_t npairs;
  const int64_t* pairs;
  int64_t chunk;
  int reset_each_chunk;
  double *y, *final_state, *boundary;
  int nthreads;
  int tid;
  int status;
} oracle_job;

static void run_pair(const oracle_job* j, int64_t slot, int64_t pair, double* h) {
  const int64_t L = j->L, H = j->H, P = j->P, N = j->N, G = j->G;
  const int64_t b = pair / H, hd = pair % H;
  const int64_t g = hd / (H / G);
  const double a = (double)j->A[hd];
  const double dskip = j->D ? (double)j->D[hd] : 0.0;
  const int64_t nc = (j->chunk > 0) ? (L + j->chunk - 1) / j->chunk : 0;

  if (j->h0) {
    const double* src = j->h0 + pair * N * P;
    for (int64_t e = 0; e < N * P; ++e) h[e] = src[e];
  } else {
    for (int64_t e = 0; e < N * P; ++e) h[e] = 0.0;
  }

  for (int64_t t = 0; t < L; ++t) {
    if (j->chunk > 0 && t % j->chunk == 0) {
      const int64_t c = t / j->chunk;
      if (j->reset_each_chunk) {
        for (int64_t e = 0; e < N * P; ++e) h[e] = 0.0;
      } else if (j->boundary) {
        double* dst = j->boundary + (slot * nc + c) * N * P;
        for (int64_t e = 0; e < N * P; ++e) dst[e] = h[e];
      }
    }
    const double dtv = (double)j->dt[(b * L + t) * H + hd];
    const double r = exp(dtv * a);
    const float* xt = j->x + ((b * L + t) * H + hd) * P;
    const float* bt = j->Bm + ((b * L + t) * G + g) * N;
    const float* ct = j->Cm + ((b * L + t) * G + g) * N;

    /* h_t = r * h_{t-1} + dt * b x^T */
    for (int64_t n = 0; n < N; ++n) {
      const double coef = dtv * (double)bt[n];
      double* hrow = h + n * P;
      for (int64_t p = 0; p < P; ++p) hrow[p] = r * hrow[p] + coef * (double)xt[p];
    }

    /* y_t = C_t^T h_t + D x_t */
    double* yt = j->y + (slot * L + t) * P;
    for (int64_t p = 0; p < P; ++p) yt[p] = dskip * (double)xt[p];
    for (int64_t n = 0; n < N; ++n) {
      const double cn = (double)ct[n];
      const double* hrow = h + n * P;
      for (int64_t p = 0; p < P; ++p) yt[p] += cn * hrow[p];
    }

    if (j->chunk > 0 && j->reset_each_chunk && j->boundary &&
        ((t + 1) % j->chunk == 0 || t + 1 == L)) {
      const int64_t c = t / j->chunk;
      double* dst = j->boundary + (slot * nc + c) * N * P;
      for (int64_t e = 0; e < N * P; ++e) dst[e] = h[e];
    }
  }
  if (j->final_state) {
    double* dst = j->final_state + slot * N * P;
    for (int64_t e = 0; e < N * P; ++e) dst[e] = h[e];
  }
}

static void* worker(void* arg) {
  oracle_job* j = (oracle_job*)arg;
  double* h = (double*)malloc(sizeof(double) * (size_t)(j->N * j->P));
  if (!h) { j->status = 3; return NULL; }
  for (int64_t s = j->tid; s < j->npairs; s += j->nthreads) {
    const int64_t pair = j->pairs ? j->pairs[s] : s;
    run_pair(j, s, pair, h);
  }
  free(h);
  return NULL;
}

/*
 * Returns 0 on success, 1 on invalid arguments, 2 on thread start failure,
 * 3 on allocation failure.
 * Layouts (all dense, row-major):
 *   x [B,L,H,P], dt [B,L,H], A [H], Bm/Cm [B,L,G,N], D [H] (may be NULL = 0),
 *   h0 [B,H,N,P] (may be NULL = zeros), pairs [npairs] of b*H+h (NULL = all,
 *   then npairs must be B*H).
 * Outputs, indexed by slot s (position in the pairs list):
 *   y [npairs,L,P], final_state [npairs,N,P] (may be NULL),
 *   boundary [npairs,ceil(L/chunk),N,P] (may be NULL; needs chunk > 0).
 */
int ssd_oracle_recurrence(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                          const float* x, const float* dt, const float* A,
                          const float* Bm, const float* Cm, const float* D,
                          const double* h0, int64_t npairs, const int64_t* pairs,
                          int64_t chunk, int reset_each_chunk,
                          double* y, double* final_state, double* boundary, int nthreads) {
  if (Bsz <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return 1;
  if (!x || !dt || !A || !Bm || !Cm || !y) return 1;
  if (!pairs && npairs != Bsz * H) return 1;
  if (boundary && chunk <= 0) return 1;
  if (pairs) {
    for (int64_t s = 0; s < npairs; ++s)
      if (pairs[s] < 0 || pairs[s] >= Bsz * H) return 1;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (npairs < nthreads) nthreads = (int)(npairs > 0 ? npairs : 1);

  oracle_job jobs[256];
  pthread_t th[256];
  int started = 0, rc = 0;
  for (int i = 0; i < nthreads; ++i) {
    oracle_job* j = &jobs[i];
    j->Bsz = Bsz; j->L = L; j->H = H; j->P = P; j->N = N; j->G = G;
    j->x = x; j->dt = dt; j->A = A; j->Bm = Bm; j->Cm = Cm; j->D = D; j->h0 = h0;
    j->npairs = npairs; j->pairs = pairs; j->chunk = chunk; j->reset_each_chunk = reset_each_chunk;
    j->y = y; j->final_state = final_state; j->boundary = boundary;
    j->nthreads = nthreads; j->tid = i; j->status = 0;
  }
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, worker, &jobs[i]) != 0) { rc = 2; break; }
    ++started;
  }
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  if (rc) return rc;
  for (int i = 0; i < nthreads; ++i)
    if (jobs[i].status) return jobs[i].status;
  return 0;
}
