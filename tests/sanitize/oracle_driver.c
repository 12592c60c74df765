/* oracle_driver.c -- runs the fp64 oracle (oracle/ssd_oracle.c, linked in)
 * under AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure).  Reads one problem from a raw file written by the test,
 * runs the recurrence with the options given on the command line, and writes
 * y, the final states and the boundary states for comparison with the
 * regular build.
 *   usage: oracle_driver IN OUT B L H P N G nthreads chunk reset npairs [pair...]
 * IN holds x, dt, A, B, C, D (float32) and h0 (float64) back to back. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ssd_oracle_recurrence(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, const float* x,
                          const float* dt, const float* A, const float* Bm, const float* Cm, const float* D,
                          const double* h0, int64_t npairs, const int64_t* pairs, int64_t chunk, int reset_each_chunk,
                          double* y, double* final_state, double* boundary, int nthreads);

static void* read_exact(FILE* f, size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p || fread(p, 1, n, f) != n) {
    fprintf(stderr, "short read\n");
    exit(2);
  }
  return p;
}

int main(int argc, char** argv) {
  if (argc < 13) return 2;
  const int64_t B = atoll(argv[3]), L = atoll(argv[4]), H = atoll(argv[5]), P = atoll(argv[6]), N = atoll(argv[7]),
                G = atoll(argv[8]);
  const int nthreads = atoi(argv[9]);
  const int64_t chunk = atoll(argv[10]);
  const int reset = atoi(argv[11]);
  int64_t npairs = atoll(argv[12]);
  int64_t* pairs = NULL;
  if (npairs > 0) {
    pairs = (int64_t*)malloc(sizeof(int64_t) * (size_t)npairs);
    for (int64_t s = 0; s < npairs; ++s) pairs[s] = atoll(argv[13 + s]);
  } else {
    npairs = B * H;
  }
  FILE* fi = fopen(argv[1], "rb");
  if (!fi) return 2;
  float* x = (float*)read_exact(fi, sizeof(float) * (size_t)(B * L * H * P));
  float* dt = (float*)read_exact(fi, sizeof(float) * (size_t)(B * L * H));
  float* A = (float*)read_exact(fi, sizeof(float) * (size_t)H);
  float* Bm = (float*)read_exact(fi, sizeof(float) * (size_t)(B * L * G * N));
  float* Cm = (float*)read_exact(fi, sizeof(float) * (size_t)(B * L * G * N));
  float* D = (float*)read_exact(fi, sizeof(float) * (size_t)H);
  double* h0 = (double*)read_exact(fi, sizeof(double) * (size_t)(B * H * N * P));
  fclose(fi);
  const int64_t nc = chunk > 0 ? (L + chunk - 1) / chunk : 0;
  double* y = (double*)malloc(sizeof(double) * (size_t)(npairs * L * P));
  double* fin = (double*)malloc(sizeof(double) * (size_t)(npairs * N * P));
  double* bnd = nc ? (double*)malloc(sizeof(double) * (size_t)(npairs * nc * N * P)) : NULL;
  const int rc = ssd_oracle_recurrence(B, L, H, P, N, G, x, dt, A, Bm, Cm, D, h0, npairs, pairs, chunk, reset, y, fin,
                                       bnd, nthreads);
  if (rc != 0) {
    fprintf(stderr, "oracle returned %d\n", rc);
    return 3;
  }
  FILE* fo = fopen(argv[2], "wb");
  if (!fo) return 2;
  fwrite(y, sizeof(double), (size_t)(npairs * L * P), fo);
  fwrite(fin, sizeof(double), (size_t)(npairs * N * P), fo);
  if (bnd) fwrite(bnd, sizeof(double), (size_t)(npairs * nc * N * P), fo);
  fclose(fo);
  free(x); free(dt); free(A); free(Bm); free(Cm); free(D); free(h0); free(y); free(fin); free(bnd); free(pairs);
  return 0;
}
