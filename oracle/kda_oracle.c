/*
 * kda_oracle.c -- plain fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package
 * smoke check and the CPU-baseline leg of the benchmark may load this
 * library.  It shares no code, header, table or helper with the HIP path,
 * and the HIP path never calls it.
 *
 * Sources (the web pages this method is described on):
 *   [DS]  docsaid.org, "Kimi Linear -- L'oubli canal par canal" (notes on
 *         arXiv 2510.26692), section "KDA : une decroissance propre a chaque
 *         canal": the GDN update (first display equation), the KDA update
 *         (second display equation) and the two-channel decay table.
 *   [GN]  fr.news.hada.io summary of the Kimi Linear report, sections
 *         "De l'attention lineaire a Gated DeltaNet" and "Algorithme
 *         parallele par chunks".
 *   [RK]  mkdocs.reaper.mx, Kimi K3 "Fondations / Attention lineaire et
 *         recurrence", sections "Le probleme de la memoire associative
 *         saturee", "Remede 1 -- La decroissance", "Remede 2 -- La regle
 *         delta", "Le calcul par blocs (chunkwise)", "Le piege numerique de
 *         la decroissance cumulee" and "Verification de comprehension".
 *
 * What is computed (per sequence and head, state S of size d_k x d_v, rows
 * indexed by key channels, multiplied from the left, [DS] KDA section):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                      (read-out after the update)
 *
 * The decay enters as g_t = log(alpha_t) (so alpha_t = exp(g_t)), one value
 * per key channel.  Everything is double precision; loops are in token
 * order with no blocking, fusion or reordering beyond what is stated at
 * each function.
 *
 * Functions:
 *   kda_oracle_recurrent   -- the definition above, token by token.
 *   kda_oracle_decode      -- one token of the same recurrence, applied to a
 *                             batch of states in place.
 *   kda_oracle_chunked     -- the chunk-parallel form ([GN] chunk algorithm,
 *                             [RK] chunkwise section), used only to check
 *                             that it equals the recurrence.
 *   kda_oracle_chunk_cumsum -- chunk-local cumulative log-decay ([RK]
 *                             cumulative-decay section).
 *   kda_oracle_ut_inverse  -- (I + A)^{-1} for strictly lower A by forward
 *                             substitution ([GN] chunk algorithm, UT
 *                             transform and forward substitution).
 *
 * Layouts (row-major, contiguous):
 *   q, k, g : [T, H, d_k]     v, o : [T, H, d_v]     beta : [T, H]
 *   S0, S_final, state : [N, H, d_k, d_v]
 *   cu_seqlens : int64 [N + 1] (cu_seqlens[0] = 0, non-decreasing,
 *                cu_seqlens[N] = T), or NULL for N sequences of T/N tokens.
 *
 * Return value: 0 on success, -1 on a bad argument, -2 on allocation
 * failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Token range [*t0, *t1) of sequence n. */
static int seq_range(const int64_t *cu_seqlens, int64_t num_seqs, int64_t T,
                     int64_t n, int64_t *t0, int64_t *t1) {
  if (cu_seqlens) {
    *t0 = cu_seqlens[n];
    *t1 = cu_seqlens[n + 1];
  } else {
    int64_t len = T / num_seqs;
    *t0 = n * len;
    *t1 = (n + 1) * len;
  }
  return (*t0 >= 0 && *t1 >= *t0 && *t1 <= T) ? 0 : -1;
}

static int check_common(const double *q, const double *k, const double *v,
                        const double *g, const double *beta,
                        const int64_t *cu_seqlens, int64_t num_seqs, int64_t T,
                        int64_t H, int64_t dk, int64_t dv) {
  if (num_seqs < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
  if (T > 0 && (!q || !k || !v || !g || !beta)) return -1;
  if (!cu_seqlens && (T % num_seqs) != 0) return -1;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  }
  return 0;
}

/*
 * One token of the recurrence on a single state S (d_k x d_v, row-major).
 *
 * [DS] KDA section, second display equation:
 *     S <- (I - beta k k^T) Diag(alpha) S + beta k v^T,   alpha = exp(g).
 * Step 1, forget ([DS] decay table; [RK] Remede 1): X = Diag(alpha) S scales
 *         row i (key channel i) by alpha_i.
 * Step 2, erase and write ([RK] Remede 2, operator form): the product
 *         (k k^T) X is evaluated as k (k^T X), so
 *         S = X - beta k (k^T X) + beta k v^T = X + k (beta (v - X^T k))^T.
 * Step 3, read-out o = S^T q on the updated state.
 * `r` is scratch of length d_v.
 */
static void kda_token(double *S, const double *q, const double *k,
                      const double *v, const double *g, double beta,
                      int64_t dk, int64_t dv, double *r, double *o) {
  for (int64_t i = 0; i < dk; ++i) {
    const double a = exp(g[i]);
    double *row = S + i * dv;
    for (int64_t j = 0; j < dv; ++j) row[j] *= a;
  }
  for (int64_t j = 0; j < dv; ++j) r[j] = 0.0;
  for (int64_t i = 0; i < dk; ++i) {
    const double ki = k[i];
    const double *row = S + i * dv;
    for (int64_t j = 0; j < dv; ++j) r[j] += row[j] * ki; /* (X^T k)_j */
  }
  for (int64_t j = 0; j < dv; ++j) r[j] = beta * (v[j] - r[j]);
  for (int64_t i = 0; i < dk; ++i) {
    const double ki = k[i];
    double *row = S + i * dv;
    for (int64_t j = 0; j < dv; ++j) row[j] += ki * r[j];
  }
  if (o) {
    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i) {
      const double qi = q[i];
      const double *row = S + i * dv;
      for (int64_t j = 0; j < dv; ++j) o[j] += row[j] * qi;
    }
  }
}

int kda_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * The recurrence, token by token, for every (sequence, head) pair.  A NULL
 * S0 means a zero initial state; S_final may be NULL.  S0 and S_final may be
 * the same buffer.  Pairs are independent, so they run in parallel.
 */
int kda_oracle_recurrent(const double *q, const double *k, const double *v,
                         const double *g, const double *beta,
                         const int64_t *cu_seqlens, int64_t num_seqs,
                         int64_t T, int64_t H, int64_t dk, int64_t dv,
                         const double *S0, double *o, double *S_final) {
  if (check_common(q, k, v, g, beta, cu_seqlens, num_seqs, T, H, dk, dv))
    return -1;
  if (T > 0 && !o) return -1;
  int err = 0;
  const int64_t pairs = num_seqs * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t n = p / H, h = p % H;
    int64_t t0, t1;
    seq_range(cu_seqlens, num_seqs, T, n, &t0, &t1);
    double *S = (double *)malloc(sizeof(double) * dk * dv);
    double *r = (double *)malloc(sizeof(double) * dv);
    if (!S || !r) {
      free(S);
      free(r);
#pragma omp atomic write
      err = -2;
      continue;
    }
    if (S0)
      memcpy(S, S0 + p * dk * dv, sizeof(double) * dk * dv);
    else
      memset(S, 0, sizeof(double) * dk * dv);
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t th = t * H + h;
      kda_token(S, q + th * dk, k + th * dk, v + th * dv, g + th * dk,
                beta[th], dk, dv, r, o + th * dv);
    }
    if (S_final) memcpy(S_final + p * dk * dv, S, sizeof(double) * dk * dv);
    free(S);
    free(r);
  }
  return err;
}

/*
 * One decode step: the recurrence applied to a single new token for each of
 * B x H states, which are updated in place.  q, k, g: [B, H, d_k];
 * v, o: [B, H, d_v]; beta: [B, H]; state: [B, H, d_k, d_v].
 */
int kda_oracle_decode(const double *q, const double *k, const double *v,
                      const double *g, const double *beta, double *state,
                      double *o, int64_t B, int64_t H, int64_t dk,
                      int64_t dv) {
  if (B < 1 || H < 1 || dk < 1 || dv < 1) return -1;
  if (!q || !k || !v || !g || !beta || !state || !o) return -1;
  int err = 0;
  const int64_t pairs = B * H;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    double *r = (double *)malloc(sizeof(double) * dv);
    if (!r) {
#pragma omp atomic write
      err = -2;
      continue;
    }
    kda_token(state + p * dk * dv, q + p * dk, k + p * dk, v + p * dv,
              g + p * dk, beta[p], dk, dv, r, o + p * dv);
    free(r);
  }
  return err;
}

/*
 * Chunk-local cumulative log-decay ([RK], cumulative-decay section: the
 * cumulative decay gamma^{1->r} is the product of alpha_1..alpha_r inside a
 * chunk, here kept as its logarithm).  Chunks hold `chunk` tokens, start at
 * each sequence start and never straddle two sequences; the last chunk of a
 * sequence may be shorter.  out[t, h, i] = sum of g[s, h, i] over the tokens
 * s of t's chunk with s <= t.
 */
int kda_oracle_chunk_cumsum(const double *g, const int64_t *cu_seqlens,
                            int64_t num_seqs, int64_t T, int64_t H,
                            int64_t dk, int64_t chunk, double *out) {
  if (num_seqs < 1 || T < 0 || H < 1 || dk < 1 || chunk < 1) return -1;
  if (T > 0 && (!g || !out)) return -1;
  if (!cu_seqlens && (T % num_seqs) != 0) return -1;
  for (int64_t n = 0; n < num_seqs; ++n) {
    int64_t t0, t1;
    if (seq_range(cu_seqlens, num_seqs, T, n, &t0, &t1)) return -1;
    for (int64_t h = 0; h < H; ++h)
      for (int64_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int64_t t = t0; t < t1; ++t) {
          if ((t - t0) % chunk == 0) acc = 0.0;
          acc += g[(t * H + h) * dk + i];
          out[(t * H + h) * dk + i] = acc;
        }
      }
  }
  return 0;
}

/*
 * Inverse of the unit lower-triangular matrix (I + A), A strictly lower
 * (n x n, row-major; entries on and above the diagonal are ignored).
 * [GN] chunk algorithm: the inverse of a lower-triangular matrix is built
 * row by row by the forward substitution of Gaussian elimination.  From
 * (I + A) T = I:  T[i][i] = 1 and, for j < i,
 *     T[i][j] = -sum_{m=j}^{i-1} A[i][m] T[m][j].
 */
int kda_oracle_ut_inverse(const double *A, int64_t n, double *Tm) {
  if (n < 0 || (n > 0 && (!A || !Tm))) return -1;
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t j = 0; j < n; ++j) Tm[i * n + j] = (i == j) ? 1.0 : 0.0;
    for (int64_t j = 0; j < i; ++j) {
      double s = 0.0;
      for (int64_t m = j; m < i; ++m) s += A[i * n + m] * Tm[m * n + j];
      Tm[i * n + j] = -s;
    }
  }
  return 0;
}

/*
 * Chunk-parallel form, used only to check that it reproduces the recurrence
 * ([RK] chunkwise section: the block form is exact, only the order of the
 * operations changes; [GN] chunk algorithm: the previous chunk's final state
 * is the next chunk's initial state, rank-1 updates are packed in WY form,
 * the UT transform replaces the sequential updates with one triangular
 * inverse, and the output combines an inter-chunk recurrent part with an
 * intra-chunk parallel part).
 *
 * For a chunk of n tokens r = 1..n entering with state S, with
 * G_r = chunk-local cumulative log-decay (g summed over tokens 1..r) and
 * the per-token erase/write written as S_r = Diag(alpha_r) S_{r-1} +
 * k_r u_r^T, u_r = beta_r (v_r - (Diag(alpha_r) S_{r-1})^T k_r), unrolling
 * the chunk gives (each product below is a plain dense product):
 *
 *   Kt = K * exp(G)        Kh = K * exp(-G)        Qt = Q * exp(G)
 *   A[r][j]  = beta_r <Kt_r, Kh_j>  for j < r, else 0
 *   Tm       = (I + A)^{-1}                         (forward substitution)
 *   W        = Tm Diag(beta) Kt,   U = Tm Diag(beta) V      (WY factors)
 *   Unew     = U - W S                              (the u_r of the chunk)
 *   P[r][j]  = <Qt_r, Kh_j>  for j <= r, else 0
 *   O        = Qt S + P Unew
 *   S       <- Diag(exp(G_n)) S + Kend^T Unew,  Kend = K * exp(G_n - G)
 *
 * (* is the per-channel product with the row of G of the same token.)
 */
int kda_oracle_chunked(const double *q, const double *k, const double *v,
                       const double *g, const double *beta,
                       const int64_t *cu_seqlens, int64_t num_seqs, int64_t T,
                       int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                       const double *S0, double *o, double *S_final) {
  if (check_common(q, k, v, g, beta, cu_seqlens, num_seqs, T, H, dk, dv))
    return -1;
  if (chunk < 1 || (T > 0 && !o)) return -1;
  int err = 0;
  const int64_t pairs = num_seqs * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t n = p / H, h = p % H;
    int64_t t0, t1;
    seq_range(cu_seqlens, num_seqs, T, n, &t0, &t1);
    const int64_t C = chunk;
    double *S = (double *)malloc(sizeof(double) * dk * dv);
    double *G = (double *)malloc(sizeof(double) * C * dk);
    double *Kt = (double *)malloc(sizeof(double) * C * dk);
    double *Kh = (double *)malloc(sizeof(double) * C * dk);
    double *Qt = (double *)malloc(sizeof(double) * C * dk);
    double *Ke = (double *)malloc(sizeof(double) * C * dk);
    double *A = (double *)malloc(sizeof(double) * C * C);
    double *Tm = (double *)malloc(sizeof(double) * C * C);
    double *P = (double *)malloc(sizeof(double) * C * C);
    double *W = (double *)malloc(sizeof(double) * C * dk);
    double *U = (double *)malloc(sizeof(double) * C * dv);
    double *Un = (double *)malloc(sizeof(double) * C * dv);
    double *Sn = (double *)malloc(sizeof(double) * dk * dv);
    if (!S || !G || !Kt || !Kh || !Qt || !Ke || !A || !Tm || !P || !W || !U ||
        !Un || !Sn) {
#pragma omp atomic write
      err = -2;
    } else {
      if (S0)
        memcpy(S, S0 + p * dk * dv, sizeof(double) * dk * dv);
      else
        memset(S, 0, sizeof(double) * dk * dv);
      for (int64_t c0 = t0; c0 < t1; c0 += C) {
        const int64_t nr = (t1 - c0 < C) ? (t1 - c0) : C;
        /* G: chunk-local cumulative log-decay. */
        for (int64_t r = 0; r < nr; ++r) {
          const double *gr = g + ((c0 + r) * H + h) * dk;
          for (int64_t i = 0; i < dk; ++i)
            G[r * dk + i] = gr[i] + (r > 0 ? G[(r - 1) * dk + i] : 0.0);
        }
        /* Decay-scaled queries and keys. */
        for (int64_t r = 0; r < nr; ++r) {
          const double *kr = k + ((c0 + r) * H + h) * dk;
          const double *qr = q + ((c0 + r) * H + h) * dk;
          for (int64_t i = 0; i < dk; ++i) {
            const double Gi = G[r * dk + i], Gn = G[(nr - 1) * dk + i];
            Kt[r * dk + i] = kr[i] * exp(Gi);
            Kh[r * dk + i] = kr[i] * exp(-Gi);
            Qt[r * dk + i] = qr[i] * exp(Gi);
            Ke[r * dk + i] = kr[i] * exp(Gn - Gi);
          }
        }
        /* A (strictly lower) and P (lower including the diagonal). */
        for (int64_t r = 0; r < nr; ++r)
          for (int64_t j = 0; j < nr; ++j) {
            double sa = 0.0, sp = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
              sa += Kt[r * dk + i] * Kh[j * dk + i];
              sp += Qt[r * dk + i] * Kh[j * dk + i];
            }
            const double br = beta[(c0 + r) * H + h];
            A[r * nr + j] = (j < r) ? br * sa : 0.0;
            P[r * nr + j] = (j <= r) ? sp : 0.0;
          }
        kda_oracle_ut_inverse(A, nr, Tm);
        /* WY factors W = Tm Diag(beta) Kt and U = Tm Diag(beta) V. */
        for (int64_t r = 0; r < nr; ++r) {
          for (int64_t i = 0; i < dk; ++i) {
            double s = 0.0;
            for (int64_t j = 0; j < nr; ++j)
              s += Tm[r * nr + j] * beta[(c0 + j) * H + h] * Kt[j * dk + i];
            W[r * dk + i] = s;
          }
          for (int64_t c = 0; c < dv; ++c) {
            double s = 0.0;
            for (int64_t j = 0; j < nr; ++j)
              s += Tm[r * nr + j] * beta[(c0 + j) * H + h] *
                   v[((c0 + j) * H + h) * dv + c];
            U[r * dv + c] = s;
          }
        }
        /* Unew = U - W S. */
        for (int64_t r = 0; r < nr; ++r)
          for (int64_t c = 0; c < dv; ++c) {
            double s = 0.0;
            for (int64_t i = 0; i < dk; ++i) s += W[r * dk + i] * S[i * dv + c];
            Un[r * dv + c] = U[r * dv + c] - s;
          }
        /* O = Qt S + P Unew. */
        for (int64_t r = 0; r < nr; ++r)
          for (int64_t c = 0; c < dv; ++c) {
            double s = 0.0;
            for (int64_t i = 0; i < dk; ++i) s += Qt[r * dk + i] * S[i * dv + c];
            for (int64_t j = 0; j < nr; ++j) s += P[r * nr + j] * Un[j * dv + c];
            o[((c0 + r) * H + h) * dv + c] = s;
          }
        /* S <- Diag(exp(G_n)) S + Kend^T Unew. */
        for (int64_t i = 0; i < dk; ++i)
          for (int64_t c = 0; c < dv; ++c) {
            double s = exp(G[(nr - 1) * dk + i]) * S[i * dv + c];
            for (int64_t j = 0; j < nr; ++j) s += Ke[j * dk + i] * Un[j * dv + c];
            Sn[i * dv + c] = s;
          }
        memcpy(S, Sn, sizeof(double) * dk * dv);
      }
      if (S_final) memcpy(S_final + p * dk * dv, S, sizeof(double) * dk * dv);
    }
    free(S); free(G); free(Kt); free(Kh); free(Qt); free(Ke); free(A);
    free(Tm); free(P); free(W); free(U); free(Un); free(Sn);
  }
  return err;
}
