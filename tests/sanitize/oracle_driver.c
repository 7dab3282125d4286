/*
 * oracle_driver.c -- exercises every function of oracle/kda_oracle.c on small
 * inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py).  Packed sequences with an empty sequence, a
 * one-token sequence and ragged tails; d_k != d_v; chunk sizes that do and do
 * not divide the lengths; the argument checks.  Cross-checks the functions
 * against each other so that a sanitizer-clean run is also a correct one:
 * chunked == recurrent, decode == one-token recurrent, (I + A) T = I,
 * cumulative sums restart at chunk and sequence starts.  Exit status 0 when
 * every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_recurrent(const double *q, const double *k, const double *v, const double *g,
                         const double *beta, const int64_t *cu_seqlens, int64_t num_seqs,
                         int64_t T, int64_t H, int64_t dk, int64_t dv, const double *S0,
                         double *o, double *S_final);
int kda_oracle_chunked(const double *q, const double *k, const double *v, const double *g,
                       const double *beta, const int64_t *cu_seqlens, int64_t num_seqs,
                       int64_t T, int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                       const double *S0, double *o, double *S_final);
int kda_oracle_decode(const double *q, const double *k, const double *v, const double *g,
                      const double *beta, double *state, double *o, int64_t B, int64_t H,
                      int64_t dk, int64_t dv);
int kda_oracle_chunk_cumsum(const double *g, const int64_t *cu_seqlens, int64_t num_seqs,
                            int64_t T, int64_t H, int64_t dk, int64_t chunk, double *out);
int kda_oracle_ut_inverse(const double *A, int64_t n, double *Tm);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* splitmix64 -> [0, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

static double *fill(int64_t n, double lo, double hi) {
  double *p = malloc(sizeof(double) * (n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uniform();
  return p;
}

static void unit_rows(double *x, int64_t rows, int64_t d) {
  for (int64_t r = 0; r < rows; ++r) {
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i) s += x[r * d + i] * x[r * d + i];
    s = sqrt(s);
    for (int64_t i = 0; i < d; ++i) x[r * d + i] /= s;
  }
}

static double maxdiff(const double *a, const double *b, int64_t n) {
  double m = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double e = fabs(a[i] - b[i]);
    if (e > m) m = e;
  }
  return m;
}

static int failures = 0;
static void check(int ok, const char *what) {
  if (!ok) {
    fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
  }
}

int main(void) {
  const int64_t H = 2, dk = 12, dv = 8, N = 4;
  const int64_t cu[5] = {0, 37, 37, 38, 100};
  const int64_t T = cu[N];
  double *q = fill(T * H * dk, -1, 1), *k = fill(T * H * dk, -1, 1);
  unit_rows(q, T * H, dk);
  unit_rows(k, T * H, dk);
  double *v = fill(T * H * dv, -1, 1), *g = fill(T * H * dk, -0.5, -0.01);
  double *beta = fill(T * H, 0.05, 0.95), *s0 = fill(N * H * dk * dv, -0.1, 0.1);
  double *o_r = calloc(T * H * dv, sizeof(double)), *s_r = calloc(N * H * dk * dv, sizeof(double));
  double *o_c = calloc(T * H * dv, sizeof(double)), *s_c = calloc(N * H * dk * dv, sizeof(double));

  check(kda_oracle_recurrent(q, k, v, g, beta, cu, N, T, H, dk, dv, s0, o_r, s_r) == 0,
        "recurrent accepts packed sequences");
  const int64_t chunks[4] = {1, 7, 16, 64};
  for (int c = 0; c < 4; ++c) {
    memset(o_c, 0, sizeof(double) * T * H * dv);
    check(kda_oracle_chunked(q, k, v, g, beta, cu, N, T, H, dk, dv, chunks[c], s0, o_c, s_c) == 0,
          "chunked accepts packed sequences");
    check(maxdiff(o_c, o_r, T * H * dv) < 1e-12, "chunked o == recurrent o");
    check(maxdiff(s_c, s_r, N * H * dk * dv) < 1e-12, "chunked S == recurrent S");
  }
  /* the empty sequence keeps its initial state */
  check(maxdiff(s_r + 1 * H * dk * dv, s0 + 1 * H * dk * dv, H * dk * dv) == 0.0,
        "empty sequence returns its initial state");
  /* in place: S0 and S_final the same buffer */
  double *s_ip = malloc(sizeof(double) * N * H * dk * dv);
  memcpy(s_ip, s0, sizeof(double) * N * H * dk * dv);
  check(kda_oracle_recurrent(q, k, v, g, beta, cu, N, T, H, dk, dv, s_ip, o_c, s_ip) == 0,
        "recurrent in place");
  check(maxdiff(s_ip, s_r, N * H * dk * dv) == 0.0, "in-place state == out-of-place state");
  /* equal lengths (no cu_seqlens), no initial state */
  check(kda_oracle_recurrent(q, k, v, g, beta, NULL, 2, T, H, dk, dv, NULL, o_r, s_r) == 0,
        "recurrent, equal lengths");
  check(kda_oracle_chunked(q, k, v, g, beta, NULL, 2, T, H, dk, dv, 16, NULL, o_c, s_c) == 0,
        "chunked, equal lengths");
  check(maxdiff(o_c, o_r, T * H * dv) < 1e-12, "chunked == recurrent, equal lengths");

  /* decode: one token per state == a one-token recurrence */
  {
    const int64_t B = 3;
    double *st = malloc(sizeof(double) * B * H * dk * dv), *od = malloc(sizeof(double) * B * H * dv);
    memcpy(st, s0, sizeof(double) * B * H * dk * dv);
    check(kda_oracle_decode(q, k, v, g, beta, st, od, B, H, dk, dv) == 0, "decode");
    const int64_t cu1[4] = {0, 1, 2, 3};
    double *o1 = malloc(sizeof(double) * B * H * dv), *s1 = malloc(sizeof(double) * B * H * dk * dv);
    check(kda_oracle_recurrent(q, k, v, g, beta, cu1, B, B, H, dk, dv, s0, o1, s1) == 0,
          "one-token recurrence");
    check(maxdiff(od, o1, B * H * dv) < 1e-14, "decode o == one-token recurrence o");
    check(maxdiff(st, s1, B * H * dk * dv) < 1e-14, "decode S == one-token recurrence S");
    free(st); free(od); free(o1); free(s1);
  }

  /* chunk-local cumulative sum restarts at chunk and sequence starts */
  {
    double *cs = malloc(sizeof(double) * T * H * dk);
    check(kda_oracle_chunk_cumsum(g, cu, N, T, H, dk, 16, cs) == 0, "chunk_cumsum");
    const int64_t starts[6] = {0, 16, 32, 37, 38, 54};
    for (int s = 0; s < 6; ++s)
      for (int64_t i = 0; i < H * dk; ++i)
        check(cs[starts[s] * H * dk + i] == g[starts[s] * H * dk + i], "cumsum restarts");
    for (int64_t i = 0; i < H * dk; ++i)
      check(fabs(cs[2 * H * dk + i] - (g[i] + g[H * dk + i] + g[2 * H * dk + i])) < 1e-15,
            "cumsum adds within a chunk");
    free(cs);
  }

  /* UT inverse: (I + A) T = I */
  {
    const int64_t n = 13;
    double *A = fill(n * n, -0.3, 0.3), *Tm = malloc(sizeof(double) * n * n);
    check(kda_oracle_ut_inverse(A, n, Tm) == 0, "ut_inverse");
    double worst = 0.0;
    for (int64_t i = 0; i < n; ++i)
      for (int64_t j = 0; j < n; ++j) {
        double s = Tm[i * n + j];
        for (int64_t m = 0; m < i; ++m) s += A[i * n + m] * Tm[m * n + j];
        const double e = fabs(s - (i == j ? 1.0 : 0.0));
        if (e > worst) worst = e;
      }
    check(worst < 1e-13, "(I + A) T == I");
    free(A); free(Tm);
  }

  /* argument checks */
  {
    const int64_t bad_cu[5] = {0, 40, 30, 38, 100};
    const int64_t bad_end[5] = {0, 37, 37, 38, 99};
    check(kda_oracle_recurrent(q, k, v, g, beta, bad_cu, N, T, H, dk, dv, NULL, o_r, NULL) != 0,
          "decreasing cu_seqlens rejected");
    check(kda_oracle_recurrent(q, k, v, g, beta, bad_end, N, T, H, dk, dv, NULL, o_r, NULL) != 0,
          "cu_seqlens not ending at T rejected");
    check(kda_oracle_recurrent(q, k, v, g, beta, NULL, 3, T, H, dk, dv, NULL, o_r, NULL) != 0,
          "T not divisible by num_seqs rejected");
    check(kda_oracle_recurrent(NULL, k, v, g, beta, cu, N, T, H, dk, dv, NULL, o_r, NULL) != 0,
          "NULL q rejected");
    check(kda_oracle_chunked(q, k, v, g, beta, cu, N, T, H, dk, dv, 0, NULL, o_c, NULL) != 0,
          "chunk size 0 rejected");
    check(kda_oracle_recurrent(q, k, v, g, beta, NULL, 1, 0, H, dk, dv, NULL, NULL, s_r) == 0,
          "zero tokens accepted");
  }

  free(q); free(k); free(v); free(g); free(beta); free(s0);
  free(o_r); free(s_r); free(o_c); free(s_c); free(s_ip);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle driver: all checks passed\n");
  return 0;
}
