// kda_backward.hip -- gradients of the chunked prefill for training.
//
// The chunk form of the forward (fr.news.hada.io Kimi Linear summary,
// section "Algorithme parallele par chunks": UT transform and WY factors,
// chosen so that training runs on the matrix units), per chunk of n <= C
// tokens with start state S, G the chunk-local cumulative log-decay and
// G_n its total:
//   Kt = K e^G, Kh = K e^-G, Qt = Q e^G, Ke = K e^(G_n - G), gam = e^G_n
//   M = Kt Kh^T, A = strict_lower(Diag(beta) M), T = (I + A)^-1
//   W = T Diag(beta) Kt, U = T Diag(beta) V, P = lower(Qt Kh^T)
//   Unew = U - W S,  O = Qt S + P Unew,  S_next = Diag(gam) S + Ke^T Unew
// is differentiated backwards, given dO and the gradient dS_next of the
// state after the chunk:
//   dUnew = P^T dO + Ke dS_next
//   dS    = Diag(gam) dS_next + Qt^T dO - W^T dUnew       (state chain)
//   dP = lower(dO Unew^T), dQt = dO S^T + dP Kh, dKe = Unew dS_next^T,
//   dgam = rowsum(dS_next * S), dW = -dUnew S^T,
//   dT = dW (Diag(beta) Kt)^T + dUnew (Diag(beta) V)^T,
//   d(Diag(beta) Kt) = T^T dW, d(Diag(beta) V) = T^T dUnew,
//   dA = strict_lower(-T^T dT T^T), dM = Diag(beta) dA,
//   dKt = Diag(beta) T^T dW + dM Kh, dKh = dM^T Kt + dP^T Qt,
//   dbeta = rowsum(dA * M + (T^T dW) * Kt + (T^T dUnew) * V),
//   dK = dKt e^G + dKh e^-G + dKe e^(G_n - G), dQ = dQt e^G, dV = Diag(beta) T^T dUnew,
//   dG = dKt*Kt - dKh*Kh + dQt*Qt - dKe*Ke, dG_n = colsum(dKe*Ke) + dgam*gam,
//   dg_s = sum_{r >= s} dG_r + dG_n.
//
// Four launches, all in fp32 over a per-tile fp32 workspace (BwdLayout):
//   bwd_prep_kernel   per (chunk, head): G, Kt, Kh, Qt, Ke, gam, M, P, T, W, U
//   bwd_state_kernel  per (sequence, head, 16-column slice): chunk start states
//   bwd_dstate_kernel per (sequence, head, 16-column slice), chunks in reverse:
//                     dS_next per chunk, dUnew, and the initial-state gradient
//   bwd_grad_kernel   per (chunk, head): dq, dk, dv, dg, dbeta
// The state columns never mix (in the forward and in dS), which is what makes
// the column slices of the two chains exact.  Rows past a chunk's end are
// zero (beta = 0, q = k = v = 0, dO = 0) and contribute nothing.  Products are
// plain fp32 loops over L2-resident tiles.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

// out[i][j] (+)= alpha * sum_k A(i, k) B(k, j) for i < M, j < N, with
// A(i, k) = TA ? A[k][i] : A[i][k] and B(k, j) = TB ? B[j][k] : B[k][j]
// (row-major, leading dimensions given).  Every thread of the block takes
// output elements in turn; callers separate dependent products with
// __syncthreads().
template <bool TA, bool TB>
__device__ void bgemm(float *out, int ldo, const float *A, int lda, const float *B, int ldb,
                      int M, int N, int K, float alpha, bool acc) {
  for (int e = threadIdx.x; e < M * N; e += blockDim.x) {
    const int i = e / N, j = e % N;
    float s = 0.f;
    for (int kk = 0; kk < K; ++kk)
      s += (TA ? A[kk * lda + i] : A[i * lda + kk]) * (TB ? B[j * ldb + kk] : B[kk * ldb + j]);
    out[i * ldo + j] = alpha * s + (acc ? out[i * ldo + j] : 0.f);
  }
}

struct TilePtr {
  float *kt, *kh, *qt, *ke, *w, *u, *vr, *gc, *tm, *pm, *mm, *gam, *bt;
};

__device__ TilePtr tile_ptrs(const BwdLayout &L, char *ws, int64_t tile, int C, int D) {
  const int64_t cd = (int64_t)C * D, cc = (int64_t)C * C;
  TilePtr p;
  p.kt = reinterpret_cast<float *>(ws + L.kt) + tile * cd;
  p.kh = reinterpret_cast<float *>(ws + L.kh) + tile * cd;
  p.qt = reinterpret_cast<float *>(ws + L.qt) + tile * cd;
  p.ke = reinterpret_cast<float *>(ws + L.ke) + tile * cd;
  p.w = reinterpret_cast<float *>(ws + L.w) + tile * cd;
  p.u = reinterpret_cast<float *>(ws + L.u) + tile * cd;
  p.vr = reinterpret_cast<float *>(ws + L.vr) + tile * cd;
  p.gc = reinterpret_cast<float *>(ws + L.gc) + tile * cd;
  p.tm = reinterpret_cast<float *>(ws + L.tm) + tile * cc;
  p.pm = reinterpret_cast<float *>(ws + L.pm) + tile * cc;
  p.mm = reinterpret_cast<float *>(ws + L.mm) + tile * cc;
  p.gam = reinterpret_cast<float *>(ws + L.gam) + tile * D;
  p.bt = reinterpret_cast<float *>(ws + L.bt) + tile * C;
  return p;
}

// Chunk range of sequence `seq`: first chunk id and chunk count.
__device__ void seq_chunks(int seq, const int *cu, int seq_len, int C, const int *seq_first,
                           int *first, int *nch, int *len) {
  int l, f;
  if (cu) {
    l = cu[seq + 1] - cu[seq];
    f = l > 0 ? seq_first[seq] : 0;
  } else {
    l = seq_len;
    f = seq * ((seq_len + C - 1) / C);
  }
  *first = f;
  *nch = (l + C - 1) / C;
  *len = l;
}

}  // namespace

// ---- 1. per-tile recompute ------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int *__restrict__ cu,
    int N, int H, int seq_len, int C, int D, BwdLayout L, char *ws) {
  __shared__ int s_loc[4];
  __shared__ int s_scan[256];
  const int h = (int)(blockIdx.x % (unsigned)H), c = (int)(blockIdx.x / (unsigned)H);
  int *seq_first = reinterpret_cast<int *>(ws + L.seq_first);
  locate_chunk(c, h, cu, N, seq_len, C, s_loc, s_scan, seq_first);
  const int t0 = s_loc[1], n = s_loc[2];
  if (n == 0) return;
  const int64_t tile = (int64_t)c * H + h;
  const TilePtr p = tile_ptrs(L, ws, tile, C, D);
  const int tid = threadIdx.x;
  const int64_t rs = (int64_t)H * D;
  // cumulative log-decay per channel (rows past the end add nothing)
  for (int i = tid; i < D; i += blockDim.x) {
    float run = 0.f;
    for (int r = 0; r < C; ++r) {
      if (r < n) run += g[(int64_t)(t0 + r) * rs + (int64_t)h * D + i];
      p.gc[r * D + i] = run;
    }
    p.gam[i] = __expf(run);
  }
  for (int r = tid; r < C; r += blockDim.x) p.bt[r] = r < n ? beta[(int64_t)(t0 + r) * H + h] : 0.f;
  __syncthreads();
  for (int e = tid; e < C * D; e += blockDim.x) {
    const int r = e / D, i = e % D;
    const bool live = r < n;
    const int64_t at = (int64_t)(t0 + r) * rs + (int64_t)h * D + i;
    const float qv = live ? to_f32(q[at]) : 0.f, kv = live ? to_f32(k[at]) : 0.f;
    const float vv = live ? to_f32(v[at]) : 0.f;
    const float G = p.gc[e], Gn = p.gc[(C - 1) * D + i];
    p.kt[e] = kv * __expf(G);
    p.kh[e] = kv * __expf(-G);
    p.qt[e] = qv * __expf(G);
    p.ke[e] = kv * __expf(Gn - G);
    p.vr[e] = vv;
  }
  __syncthreads();
  bgemm<false, true>(p.mm, C, p.kt, D, p.kh, D, C, C, D, 1.f, false);  // M = Kt Kh^T
  bgemm<false, true>(p.pm, C, p.qt, D, p.kh, D, C, C, D, 1.f, false);  // Qt Kh^T
  __syncthreads();
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int r = e / C, s = e % C;
    if (s > r) p.pm[e] = 0.f;  // P = lower incl. diagonal
  }
  // T = (I + A)^-1, A = strict_lower(beta_r M_rs): column j by thread j,
  // forward substitution row by row
  for (int j = tid; j < C; j += blockDim.x) {
    for (int r = 0; r < C; ++r) {
      float t;
      if (r < j) {
        t = 0.f;
      } else if (r == j) {
        t = 1.f;
      } else {
        float s = 0.f;
        for (int m = j; m < r; ++m) s += p.bt[r] * p.mm[r * C + m] * p.tm[m * C + j];
        t = -s;
      }
      p.tm[r * C + j] = t;
    }
  }
  __syncthreads();
  // W = T Diag(beta) Kt, U = T Diag(beta) V
  for (int e = tid; e < C * D; e += blockDim.x) {
    const int r = e / D, i = e % D;
    float sw = 0.f, su = 0.f;
    for (int m = 0; m <= r; ++m) {
      const float tb = p.tm[r * C + m] * p.bt[m];
      sw += tb * p.kt[m * D + i];
      su += tb * p.vr[m * D + i];
    }
    p.w[e] = sw;
    p.u[e] = su;
  }
}

// ---- 2. chunk start states ------------------------------------------------
// One block per (sequence, head, 16-column slice); the slice of S lives in LDS.
__global__ __launch_bounds__(256) void bwd_state_kernel(
    const int *__restrict__ cu, int N, int H, int seq_len, int C, int D,
    const float *__restrict__ s0, BwdLayout L, char *ws) {
  __shared__ float sS[128 * 16];
  __shared__ float sU[64 * 16];
  const int NS = D / 16;
  const int slice = blockIdx.x % NS, pair = blockIdx.x / NS;
  const int seq = pair / H, h = pair % H;
  if (seq >= N) return;
  const int col0 = slice * 16, tid = threadIdx.x;
  int first, nch, len;
  seq_chunks(seq, cu, seq_len, C, reinterpret_cast<const int *>(ws + L.seq_first), &first,
             &nch, &len);
  for (int e = tid; e < D * 16; e += blockDim.x) {
    const int i = e / 16, j = e % 16;
    sS[e] = s0 ? s0[((int64_t)pair * D + i) * D + col0 + j] : 0.f;
  }
  __syncthreads();
  for (int ci = 0; ci < nch; ++ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    float *sc = reinterpret_cast<float *>(ws + L.sc) + tile * D * D;
    for (int e = tid; e < D * 16; e += blockDim.x) {
      const int i = e / 16, j = e % 16;
      sc[i * D + col0 + j] = sS[e];
    }
    for (int e = tid; e < C * 16; e += blockDim.x) {  // Unew = U - W S
      const int r = e / 16, j = e % 16;
      float s = p.u[r * D + col0 + j];
      for (int i = 0; i < D; ++i) s -= p.w[r * D + i] * sS[i * 16 + j];
      sU[e] = s;
    }
    __syncthreads();
    for (int e = tid; e < D * 16; e += blockDim.x) {  // S = Diag(gam) S + Ke^T Unew
      const int i = e / 16, j = e % 16;
      float s = p.gam[i] * sS[e];
      for (int r = 0; r < C; ++r) s += p.ke[r * D + i] * sU[r * 16 + j];
      sS[e] = s;
    }
    __syncthreads();
  }
}

// ---- 3. state gradients, chunks in reverse ---------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_dstate_kernel(
    const T *__restrict__ d_o, const int *__restrict__ cu, int N, int H, int seq_len, int C,
    int D, const float *__restrict__ dsf, float *__restrict__ ds0, BwdLayout L, char *ws) {
  __shared__ float sD[128 * 16];
  __shared__ float sO[64 * 16];
  __shared__ float sU[64 * 16];
  const int NS = D / 16;
  const int slice = blockIdx.x % NS, pair = blockIdx.x / NS;
  const int seq = pair / H, h = pair % H;
  if (seq >= N) return;
  const int col0 = slice * 16, tid = threadIdx.x;
  const int64_t rs = (int64_t)H * D;
  int first, nch, len;
  seq_chunks(seq, cu, seq_len, C, reinterpret_cast<const int *>(ws + L.seq_first), &first,
             &nch, &len);
  const int t_seq = cu ? cu[seq] : seq * seq_len;
  for (int e = tid; e < D * 16; e += blockDim.x) {
    const int i = e / 16, j = e % 16;
    sD[e] = dsf ? dsf[((int64_t)pair * D + i) * D + col0 + j] : 0.f;
  }
  __syncthreads();
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    float *dse = reinterpret_cast<float *>(ws + L.dse) + tile * D * D;
    float *dun = reinterpret_cast<float *>(ws + L.dun) + tile * C * D;
    const int t0 = t_seq + ci * C, n = min(C, len - ci * C);
    for (int e = tid; e < D * 16; e += blockDim.x) {
      const int i = e / 16, j = e % 16;
      dse[i * D + col0 + j] = sD[e];
    }
    for (int e = tid; e < C * 16; e += blockDim.x) {
      const int r = e / 16, j = e % 16;
      sO[e] = r < n ? to_f32(d_o[(int64_t)(t0 + r) * rs + (int64_t)h * D + col0 + j]) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < C * 16; e += blockDim.x) {  // dUnew = P^T dO + Ke dS
      const int r = e / 16, j = e % 16;
      float s = 0.f;
      for (int m = 0; m < C; ++m) s += p.pm[m * C + r] * sO[m * 16 + j];
      for (int i = 0; i < D; ++i) s += p.ke[r * D + i] * sD[i * 16 + j];
      sU[e] = s;
      dun[r * D + col0 + j] = s;
    }
    __syncthreads();
    for (int e = tid; e < D * 16; e += blockDim.x) {  // dS = gam dS + Qt^T dO - W^T dUnew
      const int i = e / 16, j = e % 16;
      float s = p.gam[i] * sD[e];
      for (int r = 0; r < C; ++r) s += p.qt[r * D + i] * sO[r * 16 + j] - p.w[r * D + i] * sU[r * 16 + j];
      sD[e] = s;
    }
    __syncthreads();
  }
  if (ds0) {
    for (int e = tid; e < D * 16; e += blockDim.x) {
      const int i = e / 16, j = e % 16;
      ds0[((int64_t)pair * D + i) * D + col0 + j] = sD[e];
    }
  }
}

// ---- 4. per-tile gradients -------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_grad_kernel(
    const T *__restrict__ d_o, const int *__restrict__ cu, int N, int H, int seq_len, int C,
    int D, T *__restrict__ dq, T *__restrict__ dk, T *__restrict__ dv, float *__restrict__ dg,
    float *__restrict__ dbeta, BwdLayout L, char *ws) {
  __shared__ int s_loc[4];
  __shared__ int s_scan[256];
  const int h = (int)(blockIdx.x % (unsigned)H), c = (int)(blockIdx.x / (unsigned)H);
  int *seq_first = reinterpret_cast<int *>(ws + L.seq_first);
  locate_chunk(c, h, cu, N, seq_len, C, s_loc, s_scan, seq_first);
  const int t0 = s_loc[1], n = s_loc[2];
  if (n == 0) return;
  const int64_t tile = (int64_t)c * H + h;
  const TilePtr p = tile_ptrs(L, ws, tile, C, D);
  const int64_t cd = (int64_t)C * D, cc = (int64_t)C * C;
  const float *sc = reinterpret_cast<const float *>(ws + L.sc) + tile * D * D;
  const float *dse = reinterpret_cast<const float *>(ws + L.dse) + tile * D * D;
  const float *dun = reinterpret_cast<const float *>(ws + L.dun) + tile * cd;
  float *x = reinterpret_cast<float *>(ws + L.scratch) + tile * L.scratch_per_tile;
  float *unew = x, *dot = x + cd, *dqt = x + 2 * cd, *dke = x + 3 * cd, *dw = x + 4 * cd;
  float *dbkt = x + 5 * cd, *dbv = x + 6 * cd, *dkt = x + 7 * cd, *dkh = x + 8 * cd;
  float *dp = x + 9 * cd, *dt = dp + cc, *xm = dp + 2 * cc, *da = dp + 3 * cc;
  float *dgam = da + cc;
  const int tid = threadIdx.x;
  const int64_t rs = (int64_t)H * D;
  for (int e = tid; e < C * D; e += blockDim.x) {
    const int r = e / D, i = e % D;
    dot[e] = r < n ? to_f32(d_o[(int64_t)(t0 + r) * rs + (int64_t)h * D + i]) : 0.f;
  }
  // Unew = U - W S
  for (int e = tid; e < C * D; e += blockDim.x) {
    const int r = e / D, j = e % D;
    float s = p.u[e];
    for (int i = 0; i < D; ++i) s -= p.w[r * D + i] * sc[i * D + j];
    unew[e] = s;
  }
  for (int i = tid; i < D; i += blockDim.x) {  // dgam = rowsum(dS_next * S)
    float s = 0.f;
    for (int j = 0; j < D; ++j) s += dse[i * D + j] * sc[i * D + j];
    dgam[i] = s;
  }
  __syncthreads();
  bgemm<false, true>(dp, C, dot, D, unew, D, C, C, D, 1.f, false);       // dO Unew^T
  bgemm<false, true>(dqt, D, dot, D, sc, D, C, D, D, 1.f, false);        // dO S^T
  bgemm<false, true>(dke, D, unew, D, dse, D, C, D, D, 1.f, false);      // Unew dS_next^T
  bgemm<false, true>(dw, D, dun, D, sc, D, C, D, D, -1.f, false);        // -dUnew S^T
  __syncthreads();
  for (int e = tid; e < C * C; e += blockDim.x)
    if (e % C > e / C) dp[e] = 0.f;  // dP lower incl. diagonal
  __syncthreads();
  bgemm<false, false>(dqt, D, dp, C, p.kh, D, C, D, C, 1.f, true);       // + dP Kh
  // dT = dW (beta Kt)^T + dUnew (beta V)^T
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int r = e / C, s = e % C;
    float a = 0.f;
    for (int i = 0; i < D; ++i) a += dw[r * D + i] * p.kt[s * D + i] + dun[r * D + i] * p.vr[s * D + i];
    dt[e] = p.bt[s] * a;
  }
  bgemm<true, false>(dbkt, D, p.tm, C, dw, D, C, D, C, 1.f, false);      // T^T dW
  bgemm<true, false>(dbv, D, p.tm, C, dun, D, C, D, C, 1.f, false);      // T^T dUnew
  __syncthreads();
  bgemm<true, false>(xm, C, p.tm, C, dt, C, C, C, C, 1.f, false);        // T^T dT
  __syncthreads();
  bgemm<false, true>(da, C, xm, C, p.tm, C, C, C, C, -1.f, false);       // -T^T dT T^T
  __syncthreads();
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int r = e / C, s = e % C;
    if (s >= r) da[e] = 0.f;  // strictly lower
  }
  __syncthreads();
  // dKt = beta dBKt + dM Kh, dKh = dM^T Kt + dP^T Qt, dM = Diag(beta) dA
  for (int e = tid; e < C * D; e += blockDim.x) {
    const int r = e / D, i = e % D;
    float a = 0.f, b = 0.f;
    for (int s = 0; s < C; ++s) {
      a += p.bt[r] * da[r * C + s] * p.kh[s * D + i];
      b += p.bt[s] * da[s * C + r] * p.kt[s * D + i] + dp[s * C + r] * p.qt[s * D + i];
    }
    dkt[e] = p.bt[r] * dbkt[e] + a;
    dkh[e] = b;
  }
  __syncthreads();
  // outputs per row: dq, dk, dv, dbeta
  for (int e = tid; e < C * D; e += blockDim.x) {
    const int r = e / D, i = e % D;
    if (r >= n) continue;
    const float G = p.gc[e], Gn = p.gc[(C - 1) * D + i];
    const int64_t at = (int64_t)(t0 + r) * rs + (int64_t)h * D + i;
    dq[at] = from_f32<T>(dqt[e] * __expf(G));
    dk[at] = from_f32<T>(dkt[e] * __expf(G) + dkh[e] * __expf(-G) + dke[e] * __expf(Gn - G));
    dv[at] = from_f32<T>(p.bt[r] * dbv[e]);
  }
  for (int r = tid; r < n; r += blockDim.x) {
    float s = 0.f;
    for (int m = 0; m < C; ++m) s += da[r * C + m] * p.mm[r * C + m];
    for (int i = 0; i < D; ++i) s += dbkt[r * D + i] * p.kt[r * D + i] + dbv[r * D + i] * p.vr[r * D + i];
    dbeta[(int64_t)(t0 + r) * H + h] = s;
  }
  // dg: reverse cumulative sum of dG over the chunk plus dG_n, per channel
  for (int i = tid; i < D; i += blockDim.x) {
    float dgn = dgam[i] * p.gam[i];
    for (int r = 0; r < C; ++r) dgn += dke[r * D + i] * p.ke[r * D + i];
    float run = dgn;
    for (int r = n - 1; r >= 0; --r) {
      const int e = r * D + i;
      run += dkt[e] * p.kt[e] - dkh[e] * p.kh[e] + dqt[e] * p.qt[e] - dke[e] * p.ke[e];
      dg[(int64_t)(t0 + r) * rs + (int64_t)h * D + i] = run;
    }
  }
}

template <typename T>
static hipError_t launch_bwd_t(const BwdArgs &a) {
  const unsigned tiles = (unsigned)(a.grid_chunks * a.num_heads);
  const unsigned slices = (unsigned)(a.num_seqs * a.num_heads * (a.d / 16));
  const T *q = reinterpret_cast<const T *>(a.q), *k = reinterpret_cast<const T *>(a.k);
  const T *v = reinterpret_cast<const T *>(a.v), *d_o = reinterpret_cast<const T *>(a.d_o);
  if (tiles > 0)
    hipLaunchKernelGGL(bwd_prep_kernel<T>, dim3(tiles), dim3(256), 0, a.stream, q, k, v, a.g,
                       a.beta, a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len, a.chunk, a.d,
                       a.lay, a.ws);
  hipLaunchKernelGGL(bwd_state_kernel, dim3(slices), dim3(256), 0, a.stream, a.cu_seqlens,
                     a.num_seqs, a.num_heads, a.seq_len, a.chunk, a.d, a.s0, a.lay, a.ws);
  hipLaunchKernelGGL(bwd_dstate_kernel<T>, dim3(slices), dim3(256), 0, a.stream, d_o,
                     a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len, a.chunk, a.d, a.dsf,
                     a.ds0, a.lay, a.ws);
  if (tiles > 0)
    hipLaunchKernelGGL(bwd_grad_kernel<T>, dim3(tiles), dim3(256), 0, a.stream, d_o,
                       a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len, a.chunk, a.d,
                       reinterpret_cast<T *>(a.dq), reinterpret_cast<T *>(a.dk),
                       reinterpret_cast<T *>(a.dv), a.dg, a.dbeta, a.lay, a.ws);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, kda_dtype dt) {
  if (a.grid_chunks == 0 && a.ds0 == nullptr) return hipSuccess;
  if (dt == KDA_DTYPE_BF16) return launch_bwd_t<bf16>(a);
  return launch_bwd_t<float>(a);
}

}  // namespace kda
