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
// zero (beta = 0, q = k = v = 0, dO = 0) and contribute nothing.  Products run
// through block_mm: K slices of both operands are staged in LDS with
// coalesced loads and every thread accumulates a register block of the
// output in fp32.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int KS = 16;  // contraction slice staged in LDS

// out[i][j] = alpha * sum_k A(i, k) B(k, j) (+ out[i][j] when acc) for
// i < M, j < N, with A(i, k) = TA ? A[k][i] : A[i][k] and
// B(k, j) = TB ? B[j][k] : B[k][j] (row-major, leading dimensions given).
// M, N, K are multiples of 16 and M, N <= 128; out may be global memory or
// LDS and must not alias A or B.  256 threads: thread (ty, tx) = (tid / 16,
// tid % 16) owns rows ty + 16 a and columns tx + 16 b.  `lds` holds
// 2 * KS * 128 floats.  Ends with a barrier, so the block may use `out` right
// after.
template <bool TA, bool TB>
__device__ void block_mm(float *out, int ldo, const float *A, int lda, const float *B, int ldb,
                         int M, int N, int K, float alpha, bool acc, float *lds) {
  float *sa = lds, *sb = lds + KS * 128;  // sa[kk][i], sb[kk][j]
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int ma = M / 16, nb = N / 16;
  float c[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) c[a][b] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KS) {
    for (int e = tid; e < M * KS; e += 256) {
      int i, kk;
      if (TA) { kk = e / M; i = e % M; } else { i = e / KS; kk = e % KS; }
      sa[kk * M + i] = TA ? A[(k0 + kk) * lda + i] : A[i * lda + k0 + kk];
    }
    for (int e = tid; e < N * KS; e += 256) {
      int j, kk;
      if (TB) { j = e / KS; kk = e % KS; } else { kk = e / N; j = e % N; }
      sb[kk * N + j] = TB ? B[j * ldb + k0 + kk] : B[(k0 + kk) * ldb + j];
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KS; ++kk) {
      float av[8], bv[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) av[a] = a < ma ? sa[kk * M + ty + 16 * a] : 0.f;
#pragma unroll
      for (int b = 0; b < 8; ++b) bv[b] = b < nb ? sb[kk * N + tx + 16 * b] : 0.f;
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) c[a][b] += av[a] * bv[b];
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (a < ma && b < nb) {
        float *o = out + (ty + 16 * a) * ldo + tx + 16 * b;
        *o = alpha * c[a][b] + (acc ? *o : 0.f);
      }
  __syncthreads();
}

// out[r] = sum_j X[r][j] Y[r][j] (+ out[r] when acc) for r < R rows of
// length L (leading dimension ld), one wavefront per row.
__device__ void row_dots(float *out, const float *X, const float *Y, int ld, int R, int L,
                         bool acc) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int r = wv; r < R; r += 4) {
    float s = 0.f;
    for (int j = lane; j < L; j += 64) s += X[r * ld + j] * Y[r * ld + j];
    s = group_sum<64>(s);
    if (lane == 0) out[r] = s + (acc ? out[r] : 0.f);
  }
  __syncthreads();
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
  __shared__ float s_mm[2 * KS * 128];
  __shared__ float s_a[64 * 65];  // A = strict_lower(beta M), for the substitution
  const int h = (int)(blockIdx.x % (unsigned)H), c = (int)(blockIdx.x / (unsigned)H);
  int *seq_first = reinterpret_cast<int *>(ws + L.seq_first);
  locate_chunk(c, h, cu, N, seq_len, C, s_loc, s_scan, seq_first);
  const int t0 = s_loc[1], n = s_loc[2];
  if (n == 0) return;
  const int64_t tile = (int64_t)c * H + h;
  const TilePtr p = tile_ptrs(L, ws, tile, C, D);
  float *bkt = reinterpret_cast<float *>(ws + L.scratch) + tile * L.scratch_per_tile;
  float *bvv = bkt + (int64_t)C * D;  // Diag(beta) Kt and Diag(beta) V (scratch)
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
    bkt[e] = p.bt[r] * kv * __expf(G);
    bvv[e] = p.bt[r] * vv;
  }
  __syncthreads();
  block_mm<false, true>(p.mm, C, p.kt, D, p.kh, D, C, C, D, 1.f, false, s_mm);  // M = Kt Kh^T
  block_mm<false, true>(p.pm, C, p.qt, D, p.kh, D, C, C, D, 1.f, false, s_mm);  // Qt Kh^T
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int r = e / C, s = e % C;
    if (s > r) p.pm[e] = 0.f;  // P = lower incl. diagonal
    s_a[r * 65 + s] = s < r ? p.bt[r] * p.mm[e] : 0.f;
  }
  __syncthreads();
  // T = (I + A)^-1: column j by thread j, forward substitution row by row
  for (int j = tid; j < C; j += blockDim.x) {
    float tcol[64];
#pragma unroll
    for (int r = 0; r < 64; ++r) tcol[r] = 0.f;
    for (int r = 0; r < C; ++r) {
      float t = r == j ? 1.f : 0.f;
      if (r > j) {
        float s = 0.f;
        for (int m = j; m < r; ++m) s += s_a[r * 65 + m] * tcol[m];
        t = -s;
      }
      tcol[r] = t;
      p.tm[r * C + j] = t;
    }
  }
  __syncthreads();
  block_mm<false, false>(p.w, D, p.tm, C, bkt, D, C, D, C, 1.f, false, s_mm);  // W = T (beta Kt)
  block_mm<false, false>(p.u, D, p.tm, C, bvv, D, C, D, C, 1.f, false, s_mm);  // U = T (beta V)
}

// ---- chain helpers ----------------------------------------------------------
// A chunk's [rows][cols] fp32 matrix, cols % 4 == 0, moved as float4 through
// registers (rows * cols / 1024 float4 per thread; at most 8 here) into LDS
// rows of stride cols + 4.
struct Stage8 {
  f32x4 r[8];
};

__device__ void stage_load(Stage8 &st, const float *src, int rows, int cols) {
  const int n4 = rows * cols / 4;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int e = threadIdx.x + 256 * m;
    if (e < n4) st.r[m] = reinterpret_cast<const f32x4 *>(src)[e];
  }
}

__device__ void stage_store(const Stage8 &st, float *dst, int rows, int cols) {
  const int n4 = rows * cols / 4, c4 = cols / 4;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int e = threadIdx.x + 256 * m;
    if (e < n4) *reinterpret_cast<f32x4 *>(dst + (e / c4) * (cols + 4) + 4 * (e % c4)) = st.r[m];
  }
}

// ---- 2. chunk start states ------------------------------------------------
// One block per (sequence, head, 16-column slice); the slice of S lives in LDS
// and each chunk's W and Ke are staged whole in LDS, the next chunk's being
// loaded into registers while this one is computed.
__global__ __launch_bounds__(256) void bwd_state_kernel(
    const int *__restrict__ cu, int N, int H, int seq_len, int C, int D,
    const float *__restrict__ s0, BwdLayout L, char *ws) {
  extern __shared__ __align__(16) float sm[];
  const int NS = D / 16, LD = D + 4;
  float *sW = sm, *sK = sW + C * LD, *sS = sK + C * LD, *sU = sS + D * 16, *sG = sU + C * 16;
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
  Stage8 rw, rk;
  if (nch > 0) {
    const TilePtr p = tile_ptrs(L, ws, (int64_t)first * H + h, C, D);
    stage_load(rw, p.w, C, D);
    stage_load(rk, p.ke, C, D);
  }
  for (int ci = 0; ci < nch; ++ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    float *sc = reinterpret_cast<float *>(ws + L.sc) + tile * D * D;
    __syncthreads();  // the previous chunk is done with sW, sK, sU
    stage_store(rw, sW, C, D);
    stage_store(rk, sK, C, D);
    for (int e = tid; e < C * 16; e += blockDim.x) sU[e] = p.u[(e / 16) * D + col0 + e % 16];
    for (int i = tid; i < D; i += blockDim.x) sG[i] = p.gam[i];
    for (int e = tid; e < D * 16; e += blockDim.x) sc[(e / 16) * D + col0 + e % 16] = sS[e];
    __syncthreads();
    if (ci + 1 < nch) {
      const TilePtr pn = tile_ptrs(L, ws, tile + H, C, D);
      stage_load(rw, pn.w, C, D);
      stage_load(rk, pn.ke, C, D);
    }
    for (int e = tid; e < C * 16; e += blockDim.x) {  // Unew = U - W S
      const int r = e / 16, j = e % 16;
      float acc = sU[e];
      for (int i = 0; i < D; ++i) acc -= sW[r * LD + i] * sS[i * 16 + j];
      sU[e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < D * 16; e += blockDim.x) {  // S = Diag(gam) S + Ke^T Unew
      const int i = e / 16, j = e % 16;
      float acc = sG[i] * sS[e];
      for (int r = 0; r < C; ++r) acc += sK[r * LD + i] * sU[r * 16 + j];
      sS[e] = acc;
    }
  }
}

// ---- 3. state gradients, chunks in reverse ---------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_dstate_kernel(
    const T *__restrict__ d_o, const int *__restrict__ cu, int N, int H, int seq_len, int C,
    int D, const float *__restrict__ dsf, float *__restrict__ ds0, BwdLayout L, char *ws) {
  extern __shared__ __align__(16) float sm[];
  const int NS = D / 16, LD = D + 4, LP = C + 4;
  float *sW = sm, *sK = sW + C * LD, *sQ = sK + C * LD, *sP = sQ + C * LD;
  float *sD = sP + C * LP, *sO = sD + D * 16, *sU = sO + C * 16, *sG = sU + C * 16;
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
  Stage8 rw, rk, rq, rp;
  if (nch > 0) {
    const TilePtr p = tile_ptrs(L, ws, (int64_t)(first + nch - 1) * H + h, C, D);
    stage_load(rw, p.w, C, D);
    stage_load(rk, p.ke, C, D);
    stage_load(rq, p.qt, C, D);
    stage_load(rp, p.pm, C, C);
  }
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    float *dse = reinterpret_cast<float *>(ws + L.dse) + tile * D * D;
    float *dun = reinterpret_cast<float *>(ws + L.dun) + tile * C * D;
    const int t0 = t_seq + ci * C, n = min(C, len - ci * C);
    __syncthreads();  // the previous chunk is done with the staged operands
    stage_store(rw, sW, C, D);
    stage_store(rk, sK, C, D);
    stage_store(rq, sQ, C, D);
    stage_store(rp, sP, C, C);
    for (int i = tid; i < D; i += blockDim.x) sG[i] = p.gam[i];
    for (int e = tid; e < D * 16; e += blockDim.x) dse[(e / 16) * D + col0 + e % 16] = sD[e];
    for (int e = tid; e < C * 16; e += blockDim.x) {
      const int r = e / 16, j = e % 16;
      sO[e] = r < n ? to_f32(d_o[(int64_t)(t0 + r) * rs + (int64_t)h * D + col0 + j]) : 0.f;
    }
    __syncthreads();
    if (ci > 0) {
      const TilePtr pn = tile_ptrs(L, ws, tile - H, C, D);
      stage_load(rw, pn.w, C, D);
      stage_load(rk, pn.ke, C, D);
      stage_load(rq, pn.qt, C, D);
      stage_load(rp, pn.pm, C, C);
    }
    for (int e = tid; e < C * 16; e += blockDim.x) {  // dUnew = P^T dO + Ke dS
      const int r = e / 16, j = e % 16;
      float acc = 0.f;
      for (int m = 0; m < C; ++m) acc += sP[m * LP + r] * sO[m * 16 + j];
      for (int i = 0; i < D; ++i) acc += sK[r * LD + i] * sD[i * 16 + j];
      sU[e] = acc;
      dun[r * D + col0 + j] = acc;
    }
    __syncthreads();
    for (int e = tid; e < D * 16; e += blockDim.x) {  // dS = gam dS + Qt^T dO - W^T dUnew
      const int i = e / 16, j = e % 16;
      float acc = sG[i] * sD[e];
      for (int r = 0; r < C; ++r) acc += sQ[r * LD + i] * sO[r * 16 + j] - sW[r * LD + i] * sU[r * 16 + j];
      sD[e] = acc;
    }
  }
  __syncthreads();
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
  __shared__ float s_mm[2 * KS * 128];
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
    unew[e] = p.u[e];
  }
  __syncthreads();
  block_mm<false, false>(unew, D, p.w, D, sc, D, C, D, D, -1.f, true, s_mm);  // U - W S
  row_dots(dgam, dse, sc, D, D, D, false);                                    // rowsum(dS_next * S)
  block_mm<false, true>(dp, C, dot, D, unew, D, C, C, D, 1.f, false, s_mm);   // dO Unew^T
  block_mm<false, true>(dqt, D, dot, D, sc, D, C, D, D, 1.f, false, s_mm);    // dO S^T
  block_mm<false, true>(dke, D, unew, D, dse, D, C, D, D, 1.f, false, s_mm);  // Unew dS_next^T
  block_mm<false, true>(dw, D, dun, D, sc, D, C, D, D, -1.f, false, s_mm);    // -dUnew S^T
  for (int e = tid; e < C * C; e += blockDim.x)
    if (e % C > e / C) dp[e] = 0.f;  // dP lower incl. diagonal
  __syncthreads();
  block_mm<false, false>(dqt, D, dp, C, p.kh, D, C, D, C, 1.f, true, s_mm);   // + dP Kh
  // dT = (dW Kt^T + dUnew V^T) Diag(beta)
  block_mm<false, true>(dt, C, dw, D, p.kt, D, C, C, D, 1.f, false, s_mm);
  block_mm<false, true>(dt, C, dun, D, p.vr, D, C, C, D, 1.f, true, s_mm);
  for (int e = tid; e < C * C; e += blockDim.x) dt[e] *= p.bt[e % C];
  __syncthreads();
  block_mm<true, false>(dbkt, D, p.tm, C, dw, D, C, D, C, 1.f, false, s_mm);  // T^T dW
  block_mm<true, false>(dbv, D, p.tm, C, dun, D, C, D, C, 1.f, false, s_mm);  // T^T dUnew
  block_mm<true, false>(xm, C, p.tm, C, dt, C, C, C, C, 1.f, false, s_mm);    // T^T dT
  block_mm<false, true>(da, C, xm, C, p.tm, C, C, C, C, -1.f, false, s_mm);   // -T^T dT T^T
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int r = e / C, s = e % C;
    if (s >= r) da[e] = 0.f;  // strictly lower
  }
  __syncthreads();
  // dbeta = rowsum(dA * M) + rowsum(dBKt * Kt) + rowsum(dBV * V), before dA
  // is scaled into dM below
  float *dbr = xm;  // [C], xm is free now
  row_dots(dbr, da, p.mm, C, C, C, false);
  row_dots(dbr, dbkt, p.kt, D, C, D, true);
  row_dots(dbr, dbv, p.vr, D, C, D, true);
  for (int e = tid; e < C * C; e += blockDim.x) da[e] *= p.bt[e / C];  // dM = Diag(beta) dA
  __syncthreads();
  // dKt = Diag(beta) dBKt + dM Kh; dKh = dM^T Kt + dP^T Qt
  block_mm<false, false>(dkt, D, da, C, p.kh, D, C, D, C, 1.f, false, s_mm);
  block_mm<true, false>(dkh, D, da, C, p.kt, D, C, D, C, 1.f, false, s_mm);
  block_mm<true, false>(dkh, D, dp, C, p.qt, D, C, D, C, 1.f, true, s_mm);
  for (int e = tid; e < C * D; e += blockDim.x) dkt[e] += p.bt[e / D] * dbkt[e];
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
  for (int r = tid; r < n; r += blockDim.x) dbeta[(int64_t)(t0 + r) * H + h] = dbr[r];
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
  const int C = a.chunk, D = a.d;
  const size_t lds_state = sizeof(float) * (2 * C * (D + 4) + D * 16 + C * 16 + D);
  const size_t lds_dstate =
      sizeof(float) * (3 * C * (D + 4) + C * (C + 4) + D * 16 + 2 * C * 16 + D);
  // the largest shapes (d = 128, C = 64): 80,384 and 135,680 bytes
  static const hipError_t a1 = hipFuncSetAttribute(
      (const void *)bwd_state_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(sizeof(float) * (2 * 64 * 132 + 128 * 16 + 64 * 16 + 128)));
  static const hipError_t a2 = hipFuncSetAttribute(
      (const void *)bwd_dstate_kernel<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(sizeof(float) * (3 * 64 * 132 + 64 * 68 + 128 * 16 + 2 * 64 * 16 + 128)));
  if (a1 != hipSuccess) return a1;
  if (a2 != hipSuccess) return a2;
  hipLaunchKernelGGL(bwd_state_kernel, dim3(slices), dim3(256), lds_state, a.stream,
                     a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len, a.chunk, a.d, a.s0,
                     a.lay, a.ws);
  hipLaunchKernelGGL(bwd_dstate_kernel<T>, dim3(slices), dim3(256), lds_dstate, a.stream, d_o,
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
