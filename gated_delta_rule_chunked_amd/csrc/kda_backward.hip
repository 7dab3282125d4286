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
// Three or four launches over a per-tile fp32 workspace (BwdLayout; with
// bf16 inputs and C >= 32 the chunk states and state gradients are stored in
// bf16, as the products that read them round them), each instantiated per
// (head dim d, chunk C) so that every loop bound and register block is a
// compile-time constant:
//   bwd_prep_kernel   per (chunk, head): G, Kt, Kh, Qt, Ke, gam, M, P, T, W, U,
//                     and the chain-independent terms X = P^T dO, Y = Qt^T dO
//   bwd_state_kernel  per (sequence, head, 16-column slice): chunk start states
//   bwd_dstate_kernel per (sequence, head, 16-column slice), chunks in reverse:
//                     dUnew = X + Ke dS_next, dS = Diag(gam) dS_next + Y - W^T dUnew;
//                     dS_next per chunk, dUnew, and the initial-state gradient
//                     (the two chains are independent; bwd_chains_kernel runs
//                     both in one launch when they fit the GPU together)
//   bwd_grad_kernel   per (chunk, head): dq, dk, dv, dg, dbeta
// The state columns never mix (in the forward and in dS), which is what makes
// the column slices of the two chains exact.  Rows past a chunk's end are
// zero (beta = 0, q = k = v = 0, dO = 0) and contribute nothing.  Every
// product runs on the fp32 matrix cores in 16 x 16 output tiles: the per-tile
// products through block_mm (K slices of both operands staged in LDS with
// 16-byte loads, the next slice in flight while the current one is used),
// the two chains on chunk operands staged whole in LDS, the next chunk's
// being loaded into registers while the current one is computed.
#include <type_traits>

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int NTC = 256;  // threads per workgroup of the chains

// Threads per workgroup of the per-tile kernels: eight wavefronts where
// every product has enough 16 x 16 tiles to share (d >= 64 and C = 64), so
// that twice as many slice loads are in flight per tile; four otherwise.
// With fewer tiles per wave the compiler places some accumulator reads
// right behind the tile-bound branch, which the assembly scan rejects.
template <int D, int C>
constexpr int bwd_threads() { return D >= 64 && C >= 64 ? 512 : 256; }

// Products of the backward, on the fp32 matrix cores.  An M x N output
// (M <= 64, N <= 128, multiples of 16) is cut into 16 x 16 tiles, tile
// t = (t / (N/16), t % (N/16)) computed by wavefront t % NW (NW wavefronts) with
// mma_f32_k16.  Operands: A(i, k) = TA ? A[k][i] : A[i][k] and
// B(k, j) = TB ? B[j][k] : B[k][j], row-major with leading dimensions a
// multiple of 4, 16-byte aligned, in global memory or LDS.  K slices of 32
// are staged in LDS with 16-byte loads (the next slice in flight while this
// one is used): A by rows and B by columns, the contraction index
// contiguous, so that each operand of a 16-deep step is one 16-byte read
// per lane.  Waves past the last tile repeat it (no branch around the
// matrix instructions) and store nothing.
template <int M, int N, int NT = 256>
struct MmTiles {
  static constexpr int NW = NT / 64;
  static_assert(M % 16 == 0 && N % 16 == 0 && M <= 64 && N <= 128, "shape");
  static constexpr int TN = N / 16, TT = (M / 16) * TN, TPW = (TT + NW - 1) / NW;
};

// LDS floats that a product with contraction K stages, for either layout
// of each operand (7,200 at most).  The products take their staging buffer
// as an array reference, so its size is checked against every product at
// compile time.
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int M, int N, int K>
constexpr int mm_lds() {
  return (M + N + 8) * ((K < 32 ? K : 32) + 4);
}

// c[q] (MmTiles<M, N, NT>::TPW accumulators) += the wave's tiles of A B
// (contraction K).  Each K slice is staged in LDS in the order its global
// rows come in, so every staging store is one 16-byte write:
//   A: sa[i][kk] = A(i, k0 + kk), row stride KS + 4, when A is read by rows
//      (TA false); sa[kk][i], row stride M + 4, when it is read transposed;
//   B: sb[j][kk] = B(k0 + kk, j), row stride KS + 4, when TB; sb[kk][j], row
//      stride N + 4, otherwise.
// A matrix-core step reads a lane's four contraction values as one 16-byte
// read in the first layouts and as four 4-byte reads in the others; the
// padding of 4 keeps both free of bank conflicts.  Ends with a barrier.
// NA = 2: two left operands A[0], A[1] (same shape and leading dimension)
// against one B, into c[0] and c[1], staging B once per slice.
// The bf16 form (BF, for bf16 inputs) of a product whose operands are both
// read along the contraction (A by rows, B transposed) with K a multiple of
// 32: each K slice of 32 is rounded to bf16 as it is staged (rows of stride
// 40, 4 banks apart over 8 rows), and a 16 x 16 tile takes one
// v_mfma_f32_16x16x32_bf16 per slice.  Accumulation stays fp32.
// Four consecutive operand values as fp32, from fp32 or bf16 storage.
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 ld4(const bf16 *p) {
  const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
  f32x4 r;
#pragma unroll
  for (int u = 0; u < 4; ++u) r[u] = (float)b[u];
  return r;
}

template <int M, int N, int K, int NA, int NT, int CAP, typename A0T, typename A1T, typename BT>
__device__ __forceinline__ void mm_accumulate_bf(f32x4 *const *c, const A0T *A0, const A1T *A1,
                                                 int lda, const BT *B, int ldb,
                                                 float (&lds)[CAP]) {
  constexpr int NW = NT / 64;
  static_assert(K % 32 == 0, "contraction");
  constexpr int KB = 32, LB = KB + 8;
  constexpr int TN = MmTiles<M, N, NT>::TN, TT = MmTiles<M, N, NT>::TT, TPW = MmTiles<M, N, NT>::TPW;
  constexpr int GA = M * KB / 4, GB = N * KB / 4;  // float4 per slice
  constexpr int QA = (GA + NT - 1) / NT, QB = (GB + NT - 1) / NT;
  constexpr int SA = M * LB, SB = N * LB;  // bf16 elements
  static_assert(2 * (NA * SA + SB) <= 4 * CAP, "the caller's LDS buffer holds the staging");
  bf16 *la = reinterpret_cast<bf16 *>(lds), *lb = la + NA * SA;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  f32x4 ra[NA][QA], rb[QB];
  auto load = [&](int k0) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int p = 0; p < QA; ++p) {
      const int f = tid + NT * p;
      if (GA % NT == 0 || f < GA)
        ra[a][p] = a == 0 ? ld4(A0 + (f / 8) * lda + k0 + 4 * (f % 8))
                          : ld4(A1 + (f / 8) * lda + k0 + 4 * (f % 8));
    }
#pragma unroll
    for (int p = 0; p < QB; ++p) {
      const int f = tid + NT * p;
      if (GB % NT == 0 || f < GB)
        rb[p] = ld4(B + (f / 8) * ldb + k0 + 4 * (f % 8));
    }
  };
  auto cvt = [](f32x4 v) {
    bf16x4 r;
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = (bf16)v[u];
    return r;
  };
  auto store = [&]() {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int p = 0; p < QA; ++p) {
      const int f = tid + NT * p;
      if (GA % NT == 0 || f < GA)
        *reinterpret_cast<bf16x4 *>(la + a * SA + (f / 8) * LB + 4 * (f % 8)) = cvt(ra[a][p]);
    }
#pragma unroll
    for (int p = 0; p < QB; ++p) {
      const int f = tid + NT * p;
      if (GB % NT == 0 || f < GB)
        *reinterpret_cast<bf16x4 *>(lb + (f / 8) * LB + 4 * (f % 8)) = cvt(rb[p]);
    }
  };
  auto frag_a = [&](int a, int rt) {
    return *reinterpret_cast<const bf16x8 *>(la + a * SA + (16 * rt + lr) * LB + 8 * lg);
  };
  auto frag_b = [&](int ct) {
    return *reinterpret_cast<const bf16x8 *>(lb + (16 * ct + lr) * LB + 8 * lg);
  };
  load(0);
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KB) {
    store();
    __syncthreads();
    if (k0 + KB < K) load(k0 + KB);  // next slice in flight during this one
    if constexpr (TN % NW == 0) {
      constexpr int TM = M / 16, CW = TN / NW;
      bf16x8 bfr[CW];
#pragma unroll
      for (int cc = 0; cc < CW; ++cc) bfr[cc] = frag_b(wv + NW * cc);
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        bf16x8 afr[TM];
#pragma unroll
        for (int rr = 0; rr < TM; ++rr) afr[rr] = frag_a(a, rr);
#pragma unroll
        for (int rr = 0; rr < TM; ++rr)
#pragma unroll
          for (int cc = 0; cc < CW; ++cc)
            c[a][rr * CW + cc] = mma_k32(afr[rr], bfr[cc], c[a][rr * CW + cc]);
      }
    } else {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int t = TT % NW == 0 ? wv + NW * q : min(wv + NW * q, TT - 1);
        c[a][q] = mma_k32(frag_a(a, t / TN), frag_b(t % TN), c[a][q]);
      }
    }
    __syncthreads();
  }
}

template <int M, int N, int K, bool TA, bool TB, int NA, bool BF = false, int NT = 256, int CAP,
          typename A0T, typename A1T, typename BT>
__device__ __forceinline__ void mm_accumulate_n(f32x4 *const *c, const A0T *A0, const A1T *A1,
                                                int lda, const BT *B, int ldb,
                                                float (&lds)[CAP]) {
  constexpr int NW = NT / 64;
  static_assert(K % 16 == 0, "contraction");
  if constexpr (BF && !TA && TB && K % 32 == 0) {
    mm_accumulate_bf<M, N, K, NA, NT>(c, A0, A1, lda, B, ldb, lds);
    return;
  }
  constexpr int KS = K < 32 ? K : 32, LK = KS + 4;  // slice depth, row stride by rows
  constexpr int LMA = M + 4, LNB = N + 4;           // row strides of the transposed layouts
  constexpr int TN = MmTiles<M, N, NT>::TN, TT = MmTiles<M, N, NT>::TT, TPW = MmTiles<M, N, NT>::TPW;
  constexpr int FA = M * KS / 4, FB = N * KS / 4;  // float4 per slice
  constexpr int PA = (FA + NT - 1) / NT, PB = (FB + NT - 1) / NT;
  constexpr int SA = TA ? KS * LMA : M * LK, SB = TB ? N * LK : KS * LNB;
  static_assert(NA == 1 || NA == 2, "one or two left operands");
  // (the bf16 form above returned already; its own check is in mm_accumulate_bf)
  static_assert((BF && !TA && TB && K % 32 == 0) ||
                    (SA + SB <= mm_lds<M, N, K>() && NA * SA + SB <= CAP &&
                     (NA > 1 || mm_lds<M, N, K>() <= CAP)),
                "the caller's LDS buffer holds this product's staging");
  float *sb = lds + NA * SA;  // A[a]'s slice at lds + a * SA
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  f32x4 ra[NA][PA], rb[PB];
  auto load = [&](int k0) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int f = tid + NT * p;
      if (FA % NT == 0 || f < FA) {
        if (TA) {
          const int kk = f / (M / 4), i4 = f % (M / 4);
          ra[a][p] = a == 0 ? ld4(A0 + (k0 + kk) * lda + 4 * i4) : ld4(A1 + (k0 + kk) * lda + 4 * i4);
        } else {
          const int i = f / (KS / 4), k4 = f % (KS / 4);
          ra[a][p] = a == 0 ? ld4(A0 + i * lda + k0 + 4 * k4) : ld4(A1 + i * lda + k0 + 4 * k4);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int f = tid + NT * p;
      if (FB % NT == 0 || f < FB) {
        if (TB) {
          const int j = f / (KS / 4), k4 = f % (KS / 4);
          rb[p] = ld4(B + j * ldb + k0 + 4 * k4);
        } else {
          const int kk = f / (N / 4), j4 = f % (N / 4);
          rb[p] = ld4(B + (k0 + kk) * ldb + 4 * j4);
        }
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      float *sa = lds + a * SA;
      const int f = tid + NT * p;
      if (FA % NT == 0 || f < FA) {
        if (TA) {
          const int kk = f / (M / 4), i4 = f % (M / 4);
          *reinterpret_cast<f32x4 *>(sa + kk * LMA + 4 * i4) = ra[a][p];
        } else {
          const int i = f / (KS / 4), k4 = f % (KS / 4);
          *reinterpret_cast<f32x4 *>(sa + i * LK + 4 * k4) = ra[a][p];
        }
      }
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int f = tid + NT * p;
      if (FB % NT == 0 || f < FB) {
        if (TB) {
          const int j = f / (KS / 4), k4 = f % (KS / 4);
          *reinterpret_cast<f32x4 *>(sb + j * LK + 4 * k4) = rb[p];
        } else {
          const int kk = f / (N / 4), j4 = f % (N / 4);
          *reinterpret_cast<f32x4 *>(sb + kk * LNB + 4 * j4) = rb[p];
        }
      }
    }
  };
  // a lane's operands of a 16-deep step: A(16 rt + lr, ks + 4 lg + u) and
  // B(ks + 4 lg + u, 16 ct + lr), u = 0 .. 3
  auto frag_a = [&](int a, int rt, int ks) -> f32x4 {
    const float *sa = lds + a * SA;
    if constexpr (TA) {
      f32x4 a;
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = sa[(ks + 4 * lg + u) * LMA + 16 * rt + lr];
      return a;
    } else {
      return *reinterpret_cast<const f32x4 *>(sa + (16 * rt + lr) * LK + ks + 4 * lg);
    }
  };
  auto frag_b = [&](int ct, int ks) -> f32x4 {
    if constexpr (TB) {
      return *reinterpret_cast<const f32x4 *>(sb + (16 * ct + lr) * LK + ks + 4 * lg);
    } else {
      f32x4 b;
#pragma unroll
      for (int u = 0; u < 4; ++u) b[u] = sb[(ks + 4 * lg + u) * LNB + 16 * ct + lr];
      return b;
    }
  };
  load(0);
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KS) {
    store();
    __syncthreads();
    if (k0 + KS < K) load(k0 + KS);  // next slice in flight during this one
#pragma unroll
    for (int ks = 0; ks < KS; ks += 16) {
      if constexpr (TN % NW == 0) {
        // wave wv owns tile columns wv + 4 cc of every tile row (q = row * CW
        // + cc, the same tiles as t = wv + 4 q): each A and B fragment is read
        // from LDS once per step and used for a whole row or column of tiles
        constexpr int TM = M / 16, CW = TN / NW;
        f32x4 bf[CW];
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) bf[cc] = frag_b(wv + NW * cc, ks);
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          f32x4 af[TM];
#pragma unroll
          for (int rr = 0; rr < TM; ++rr) af[rr] = frag_a(a, rr, ks);
#pragma unroll
          for (int rr = 0; rr < TM; ++rr)
#pragma unroll
            for (int cc = 0; cc < CW; ++cc)
              c[a][rr * CW + cc] = mma_f32_k16(af[rr], bf[cc], c[a][rr * CW + cc]);
        }
      } else {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
          const int t = TT % NW == 0 ? wv + NW * q : min(wv + NW * q, TT - 1);
          c[a][q] = mma_f32_k16(frag_a(a, t / TN, ks), frag_b(t % TN, ks), c[a][q]);
        }
      }
    }
    __syncthreads();
  }
}

// c[q] += the wave's tiles of A B (one left operand), as above.
template <int M, int N, int K, bool TA, bool TB, bool BF = false, int NT = 256, int CAP,
          typename AT, typename BT>
__device__ __forceinline__ void mm_accumulate(f32x4 *c, const AT *A, int lda, const BT *B,
                                              int ldb, float (&lds)[CAP]) {
  f32x4 *const cs[1] = {c};
  mm_accumulate_n<M, N, K, TA, TB, 1, BF, NT>(cs, A, A, lda, B, ldb, lds);
}

// out = alpha c + (init ? init : 0), tile by tile (init may be out itself;
// leading dimension ldo for both), rounded to out's type.  Ends with a barrier.
template <int M, int N, int NT = 256, typename OT, typename IT>
__device__ __forceinline__ void mm_store(OT *out, int ldo, const IT *init, float alpha,
                                         f32x4 *c) {
  constexpr int NW = NT / 64;
  constexpr int TN = MmTiles<M, N, NT>::TN, TT = MmTiles<M, N, NT>::TT, TPW = MmTiles<M, N, NT>::TPW;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the results reach ordinary registers here, in straight-line code, before
  // the branch on the tile index below
#pragma unroll
  for (int q = 0; q < TPW; ++q) asm volatile("" : "+v"(c[q]));
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int t = wv + NW * q;
    if (TT % NW == 0 || t < TT) {
      const int at = (16 * (t / TN) + 4 * lg) * ldo + 16 * (t % TN) + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[at + i * ldo] = (OT)(alpha * c[q][i] + (init ? (float)init[at + i * ldo] : 0.f));
    }
  }
  __syncthreads();
}

// out = alpha A B (+ out when acc).  `lds` holds at least mm_lds<M, N, K>()
// floats.
template <int M, int N, int K, bool TA, bool TB, bool BF = false, int NT = 256, int CAP,
          typename OT, typename AT, typename BT>
__device__ __forceinline__ void block_mm(OT *out, int ldo, const AT *A, int lda,
                                         const BT *B, int ldb, float alpha, bool acc,
                                         float (&lds)[CAP]) {
  f32x4 c[MmTiles<M, N, NT>::TPW];
#pragma unroll
  for (int q = 0; q < MmTiles<M, N, NT>::TPW; ++q) c[q] = zero4();
  mm_accumulate<M, N, K, TA, TB, BF, NT>(c, A, lda, B, ldb, lds);
  mm_store<M, N, NT>(out, ldo, acc ? out : nullptr, alpha, c);
}

// out = init + alpha A B (init has leading dimension ldo).
template <int M, int N, int K, bool TA, bool TB, bool BF = false, int NT = 256, int CAP,
          typename OT, typename AT, typename BT>
__device__ __forceinline__ void block_mm_init(OT *out, int ldo, const float *init, float alpha,
                                              const AT *A, int lda, const BT *B, int ldb,
                                              float (&lds)[CAP]) {
  f32x4 c[MmTiles<M, N, NT>::TPW];
#pragma unroll
  for (int q = 0; q < MmTiles<M, N, NT>::TPW; ++q) c[q] = zero4();
  mm_accumulate<M, N, K, TA, TB, BF, NT>(c, A, lda, B, ldb, lds);
  mm_store<M, N, NT>(out, ldo, init, alpha, c);
}

// out = A1 B1 + A2 B2, both products accumulated in registers.
template <int M, int N, int K1, bool TA1, bool TB1, int K2, bool TA2, bool TB2, bool BF = false,
          int NT = 256, int CAP, typename A1T, typename B1T, typename A2T, typename B2T>
__device__ __forceinline__ void block_mm2(float *out, int ldo, const A1T *A1, int lda1,
                                          const B1T *B1, int ldb1, const A2T *A2, int lda2,
                                          const B2T *B2, int ldb2, float (&lds)[CAP]) {
  f32x4 c[MmTiles<M, N, NT>::TPW];
#pragma unroll
  for (int q = 0; q < MmTiles<M, N, NT>::TPW; ++q) c[q] = zero4();
  mm_accumulate<M, N, K1, TA1, TB1, BF, NT>(c, A1, lda1, B1, ldb1, lds);
  mm_accumulate<M, N, K2, TA2, TB2, BF, NT>(c, A2, lda2, B2, ldb2, lds);
  mm_store<M, N, NT>(out, ldo, static_cast<const float *>(nullptr), 1.f, c);
}

// out1 = A1 B and out2 = A2 B (A1, A2 of the same shape and leading
// dimension), staging B once.
template <int M, int N, int K, bool TA, bool TB, bool BF = false, int NT = 256, int CAP,
          typename A1T, typename A2T, typename BT>
__device__ __forceinline__ void block_mm_pair(float *out1, float *out2, int ldo, const A1T *A1,
                                              const A2T *A2, int lda, const BT *B, int ldb,
                                              float (&lds)[CAP]) {
  f32x4 c1[MmTiles<M, N, NT>::TPW], c2[MmTiles<M, N, NT>::TPW];
#pragma unroll
  for (int q = 0; q < MmTiles<M, N, NT>::TPW; ++q) c1[q] = c2[q] = zero4();
  f32x4 *const cs[2] = {c1, c2};
  mm_accumulate_n<M, N, K, TA, TB, 2, BF, NT>(cs, A1, A2, lda, B, ldb, lds);
  mm_store<M, N, NT>(out1, ldo, static_cast<const float *>(nullptr), 1.f, c1);
  mm_store<M, N, NT>(out2, ldo, static_cast<const float *>(nullptr), 1.f, c2);
}

// out[r] = sum_j X[r][j] Y[r][j] (+ out[r] when acc) for r < R rows of
// length L (leading dimension ld, a multiple of 4; 16-byte aligned rows).
// TPR consecutive threads share a row, each reading float4s part, part +
// TPR, ...; a thread's rows are r0, r0 + NT / TPR, ..., all loaded before
// any of the sums is reduced.  Ends with a barrier.
template <int R, int L, int NT = 256, typename XT, typename YT>
__device__ __forceinline__ void row_dots(float *out, const XT *X, const YT *Y, int ld, bool acc) {
  constexpr int TPR = L / 4 < 16 ? L / 4 : 16;  // threads per row
  constexpr int V = L / (4 * TPR);              // float4 per thread and row
  constexpr int RPP = NT / TPR;                 // rows per pass of the block
  constexpr int NP = (R + RPP - 1) / RPP;       // passes
  static_assert(TPR >= 4 && L % (4 * TPR) == 0, "row_dots shape");
  const int part = threadIdx.x % TPR, r0 = threadIdx.x / TPR;
  float s[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int r = min(r0 + RPP * pp, R - 1);
    s[pp] = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const f32x4 x = ld4(X + r * ld + 4 * (part + TPR * v));
      const f32x4 y = ld4(Y + r * ld + 4 * (part + TPR * v));
      s[pp] += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
    }
  }
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const float t = group_sum<TPR>(s[pp]);
    const int r = r0 + RPP * pp;
    if (part == 0 && r < R) out[r] = t + (acc ? out[r] : 0.f);
  }
  __syncthreads();
}

// Rounds four fp32 values to bf16 (round to nearest even).
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (bf16)v[i];
  return r;
}

struct TilePtr {
  float *kt, *kh, *qt, *ke, *w, *u, *vr, *gc, *tm, *pm, *mm, *gam, *bt, *px, *qy;
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
  p.px = reinterpret_cast<float *>(ws + L.px) + tile * cd;
  p.qy = reinterpret_cast<float *>(ws + L.qy) + tile * (int64_t)D * D;
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
template <typename T, int D, int C>
__global__ __launch_bounds__((bwd_threads<D, C>())) void bwd_prep_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ d_o, const float *__restrict__ g, const float *__restrict__ beta,
    const int4 *__restrict__ tab, int N, int H, int seq_len, BwdLayout L, char *ws) {
  constexpr int NT = bwd_threads<D, C>();
  constexpr int LA = C + 4;
  constexpr int YM = D < 64 ? D : 64;  // row block of dO^T Qt
  constexpr int MM_PAIR = 3 * C * ((D < 32 ? D : 32) + 4);  // Kt, Qt and Kh slices together
  constexpr int MM = cmax(cmax(MM_PAIR, mm_lds<C, D, C>()),
                          cmax(mm_lds<YM, C, C>(), mm_lds<YM, D, C>()));
  __shared__ __align__(16) float s_mm[MM];
  __shared__ __align__(16) float s_a[C * LA];  // A = strict_lower(beta M), for the substitution
  __shared__ __align__(16) float s_do[C * D];  // dO, zero past the chunk's end
  const int h = (int)(blockIdx.x % (unsigned)H), c = (int)(blockIdx.x / (unsigned)H);
  const ChunkLoc loc = chunk_loc(c, tab, N, seq_len, C);
  const int t0 = loc.t0, n = loc.n;
  if (n == 0) return;
  const int64_t tile = (int64_t)c * H + h;
  const TilePtr p = tile_ptrs(L, ws, tile, C, D);
  float *tb = reinterpret_cast<float *>(ws + L.scratch) + tile * L.scratch_per_tile;  // T Diag(beta)
  const int tid = threadIdx.x;
  const int64_t rs = (int64_t)H * D;
  // cumulative log-decay per channel (rows past the end add nothing); every
  // row's load is issued before the running sum needs it
  if (tid < D) {
    const float *gp = g + (int64_t)t0 * rs + (int64_t)h * D + tid;
    float gv[C];
#pragma unroll
    for (int r = 0; r < C; ++r) gv[r] = gp[(int64_t)min(r, n - 1) * rs];
    float run = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      run += r < n ? gv[r] : 0.f;
      p.gc[r * D + tid] = run;
    }
    p.gam[tid] = __expf(run);
  }
  for (int r = tid; r < C; r += NT) p.bt[r] = r < n ? beta[(int64_t)(t0 + r) * H + h] : 0.f;
  __syncthreads();
  // For bf16 inputs Ke is needed only as the chains' bf16 copies, so its
  // row-major copy is written here (after T Diag(beta) in the scratch) and
  // no fp32 Ke is stored.
  bf16 *keb = reinterpret_cast<bf16 *>(tb + C * C) + C * D;
  // V is kept in the input type: the copy is exact, and half the bytes for bf16
  T *vr = reinterpret_cast<T *>(p.vr);
  for (int e4 = tid; e4 < C * D / 4; e4 += NT) {
    const int r = e4 / (D / 4), i = 4 * (e4 % (D / 4));
    const float live = r < n ? 1.f : 0.f;
    const int64_t at = (int64_t)(t0 + min(r, n - 1)) * rs + (int64_t)h * D + i;
    const f32x4 qv = load4_f32<T>(q + at) * live, kv = load4_f32<T>(k + at) * live;
    const f32x4 vv = load4_f32<T>(v + at) * live;
    const f32x4 ov = load4_f32<T>(d_o + at) * live;
    const f32x4 G = *reinterpret_cast<const f32x4 *>(p.gc + r * D + i);
    const f32x4 Gn = *reinterpret_cast<const f32x4 *>(p.gc + (C - 1) * D + i);
    f32x4 eg, emg, egn;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      eg[u] = __expf(G[u]);
      emg[u] = __expf(-G[u]);
      egn[u] = __expf(Gn[u] - G[u]);
    }
    const int e = r * D + i;
    *reinterpret_cast<f32x4 *>(p.kt + e) = kv * eg;
    *reinterpret_cast<f32x4 *>(p.kh + e) = kv * emg;
    *reinterpret_cast<f32x4 *>(p.qt + e) = qv * eg;
    if constexpr (sizeof(T) == 2)
      *reinterpret_cast<bf16x4 *>(keb + e) = to_bf16x4(kv * egn);
    else
      *reinterpret_cast<f32x4 *>(p.ke + e) = kv * egn;
    if constexpr (sizeof(T) == 2)
      *reinterpret_cast<bf16x4 *>(vr + e) = to_bf16x4(vv);
    else
      *reinterpret_cast<f32x4 *>(vr + e) = vv;
    *reinterpret_cast<f32x4 *>(s_do + e) = ov;
  }
  __syncthreads();
  // M = Kt Kh^T and Qt Kh^T, staging Kh once
  constexpr bool BF = sizeof(T) == 2;  // bf16 matrix cores where both operands allow
  block_mm_pair<C, C, D, false, true, BF, NT>(p.mm, p.pm, C, p.kt, p.qt, D, p.kh, D, s_mm);
  for (int e = tid; e < C * C; e += NT) {
    const int r = e / C, s = e % C;
    if (s > r) p.pm[e] = 0.f;  // P = lower incl. diagonal
    s_a[r * LA + s] = s < r ? p.bt[r] * p.mm[e] : 0.f;
  }
  __syncthreads();
  // T = (I + A)^-1 by forward substitution, column j by thread j:
  // T[r][j] = [r == j] - sum_{m < r} A[r][m] T[m][j].  Entries not yet
  // computed are still zero, so the sums run over whole 4-vectors of a row.
  if (tid < C) {
    const int j = tid;
    const float bj = p.bt[j];
    float t[C];
#pragma unroll
    for (int r = 0; r < C; ++r) t[r] = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float s = 0.f;
#pragma unroll
      for (int m4 = 0; m4 < (r + 3) / 4; ++m4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4 *>(s_a + r * LA + 4 * m4);
#pragma unroll
        for (int u = 0; u < 4; ++u) s += a4[u] * t[4 * m4 + u];
      }
      t[r] = r < j ? 0.f : (r == j ? 1.f : -s);
      p.tm[r * C + j] = t[r];
      tb[r * C + j] = t[r] * bj;
    }
  }
  __syncthreads();
  block_mm<C, D, C, false, false, false, NT>(p.w, D, tb, C, p.kt, D, 1.f, false, s_mm);  // W = (T Diag(beta)) Kt
  block_mm<C, D, C, false, false, false, NT>(p.u, D, tb, C, vr, D, 1.f, false, s_mm);  // U = (T Diag(beta)) V
  // the two terms of the state-gradient recursion that do not depend on it,
  // X = P^T dO and Y = Qt^T dO, so that its serial steps need only W and Ke.
  // They are stored transposed (X^T = dO^T P, Y^T = dO^T Qt): a chain lane's
  // four rows of one column are then one 16-byte load.
#pragma unroll
  for (int n0 = 0; n0 < D; n0 += YM) {
    block_mm<YM, C, C, true, false, false, NT>(p.px + n0 * C, C, s_do + n0, D, p.pm, C, 1.f, false, s_mm);
    block_mm<YM, D, C, true, false, false, NT>(p.qy + n0 * D, D, s_do + n0, D, p.qt, D, 1.f, false, s_mm);
  }
  if constexpr (sizeof(T) == 2) {
    // the chains' bf16 copies: W and Ke row-major and, for C >= 32, W^T and
    // Ke^T.  A thread takes 8 rows x 4 channels of each, read as 16-byte rows,
    // and writes them back as 4-wide rows and as four 8-token columns.
    __syncthreads();
    bf16 *wb = reinterpret_cast<bf16 *>(tb + C * C);
    for (int e = tid; e < C * D / 32; e += NT) {
      const int c4 = 4 * (e % (D / 4)), r8 = 8 * (e / (D / 4));
#pragma unroll
      for (int mtx = 0; mtx < 2; ++mtx) {
        bf16 *dst = wb + mtx * C * D;
        f32x4 x[8];
        if (mtx == 0) {  // W: fp32 rows, rounded here
#pragma unroll
          for (int i = 0; i < 8; ++i)
            x[i] = *reinterpret_cast<const f32x4 *>(p.w + (r8 + i) * D + c4);
#pragma unroll
          for (int i = 0; i < 8; ++i) *reinterpret_cast<bf16x4 *>(dst + (r8 + i) * D + c4) = to_bf16x4(x[i]);
        } else {  // Ke: its bf16 rows, written in the element-wise pass
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const bf16x4 b4 = *reinterpret_cast<const bf16x4 *>(dst + (r8 + i) * D + c4);
#pragma unroll
            for (int u = 0; u < 4; ++u) x[i][u] = (float)b4[u];
          }
        }
        if constexpr (C >= 32) {
          bf16 *dt = wb + (2 + mtx) * C * D;  // [D][C]
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            bf16x8 t8;
#pragma unroll
            for (int i = 0; i < 8; ++i) t8[i] = (bf16)x[i][u];
            *reinterpret_cast<bf16x8 *>(dt + (c4 + u) * C + r8) = t8;
          }
        }
      }
    }
  }
}

// ---- chain helpers ----------------------------------------------------------
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// A chunk's [R][CO] matrix, stored as fp32 or bf16, moved in 16-byte pieces
// through registers into fp32 LDS rows of stride CO + 4.  A bf16 piece holds
// 8 elements, two to a dword (low half first); widening one is a shift.
template <int R, int CO, typename WT>
struct Stage {
  static constexpr int EV = 16 / (int)sizeof(WT);  // elements per piece
  static constexpr int NV = R * CO / EV, P = (NV + NTC - 1) / NTC;
  static_assert(CO % EV == 0, "a piece stays within one row");
  u32x4 r[P];
  __device__ __forceinline__ void load(const WT *src) {
#pragma unroll
    for (int m = 0; m < P; ++m) {
      const int e = threadIdx.x + NTC * m;
      if (NV % NTC == 0 || e < NV) r[m] = reinterpret_cast<const u32x4 *>(src)[e];
    }
  }
  __device__ __forceinline__ void store(float *dst) const {
#pragma unroll
    for (int m = 0; m < P; ++m) {
      const int e = threadIdx.x + NTC * m;
      if (NV % NTC == 0 || e < NV) {
        float *at = dst + (e / (CO / EV)) * (CO + 4) + EV * (e % (CO / EV));
        if constexpr (EV == 4) {
          *reinterpret_cast<f32x4 *>(at) = __builtin_bit_cast(f32x4, r[m]);
        } else {
          f32x4 lo, hi;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            lo[2 * u] = __uint_as_float(r[m][u] << 16);
            lo[2 * u + 1] = __uint_as_float(r[m][u] & 0xffff0000u);
            hi[2 * u] = __uint_as_float(r[m][2 + u] << 16);
            hi[2 * u + 1] = __uint_as_float(r[m][2 + u] & 0xffff0000u);
          }
          *reinterpret_cast<f32x4 *>(at) = lo;
          *reinterpret_cast<f32x4 *>(at + 4) = hi;
        }
      }
    }
  }
};

// W and Ke as the two chains stream them.  For bf16 inputs they are the bf16
// copies that the per-tile pass leaves in the tile's scratch, right after
// T Diag(beta): half the bytes of each chain step, rounded as the forward's
// own chain rounds them.  The gradient pass reuses that scratch afterwards.
// For bf16 inputs and C >= 32 the chains also take W^T and Ke^T ([d][C]
// bf16, the same rounded values), which follow the two copies in scratch.
__device__ __forceinline__ void chain_operands_t(const BwdLayout &L, char *ws, int64_t tile, int C,
                                                 int D, const bf16 **wt, const bf16 **ket) {
  const float *x = reinterpret_cast<const float *>(ws + L.scratch) + tile * L.scratch_per_tile;
  *wt = reinterpret_cast<const bf16 *>(x + C * C) + 2 * C * D;
  *ket = *wt + C * D;
}

// Chains on the bf16 matrix cores: bf16 inputs with chunks of 32 or more.
template <int C, typename WT>
constexpr bool chain_bf16() { return sizeof(WT) == 2 && C >= 32; }

template <typename WT>
__device__ __forceinline__ void chain_operands(const BwdLayout &L, char *ws, int64_t tile, int C,
                                               int D, const WT **w, const WT **ke) {
  if constexpr (sizeof(WT) == 4) {
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    *w = p.w;
    *ke = p.ke;
  } else {
    const float *x = reinterpret_cast<const float *>(ws + L.scratch) + tile * L.scratch_per_tile;
    *w = reinterpret_cast<const WT *>(x + C * C);
    *ke = *w + C * D;
  }
}

// The two chains run their per-chunk products on the fp32 matrix cores in
// 16 x 16 output tiles (mma_f32_k16: lane l = 16 g + c supplies A[c][4g + i]
// and B[4g + i][c] and holds D[4g + i][c]).  Wave w owns token block w of the
// chunk (rows 16 w ..) and channel blocks w*CBW .. of the state slice.  The
// right-hand operands sit transposed in LDS (column c of the slice is a row),
// so that they are one 16-byte read per lane; a left-hand operand used
// transposed (Ke^T, W^T) is four 4-byte reads, free of bank conflicts with
// the row padding of 4.  Matrix results are read (stored or combined) in
// straight-line code right after the instructions that produce them.
template <int D, int C>
struct ChainShape {
  static constexpr int NS = D / 16, LD = D + 4, LU = C + 4;
  static constexpr int NRB = C / 16, NCB = D / 16, CBW = (NCB + 3) / 4;
};

// Chain workgroup b serves slice (b / 8) % NS of pair 8 ((b / 8) / NS) + b % 8:
// the slices of one (sequence, head) share blockIdx % 8, so they run on one
// XCD and its L2 serves each chunk's operands to all of them.  The grid is
// 8 * ceil(pairs / 8) * NS; false for a workgroup past the last pair.
template <int NS>
__device__ __forceinline__ bool chain_block(int b, int pairs, int *slice, int *pair) {
  const int local = b >> 3;
  *slice = local % NS;
  *pair = (local / NS) * 8 + (b & 7);
  return *pair < pairs;
}
inline unsigned chain_grid(int pairs, int ns) { return 8u * (unsigned)((pairs + 7) / 8) * ns; }

template <int D, int C, typename WT>
constexpr size_t state_lds_bytes() {
  using Sh = ChainShape<D, C>;
  if constexpr (chain_bf16<C, WT>())  // bf16 [C][D + 8], [D][C + 8], [16][D + 8], [16][C + 8]
    return sizeof(bf16) * ((C + 16) * (D + 8) + (D + 16) * (C + 8));
  else
    return sizeof(float) * (2 * C * Sh::LD + 16 * Sh::LD + 16 * Sh::LU);
}
template <int D, int C, typename WT>
constexpr size_t dstate_lds_bytes() {
  return state_lds_bytes<D, C, WT>();  // W, Ke, the transposed dS_next and dUnew
}

// A chunk's [R][CO] bf16 matrix moved in 16-byte pieces through registers
// into bf16 LDS rows of stride CO + 8 (rows 4 banks apart, so that the
// 16-byte fragment reads of 8 consecutive rows hit distinct banks).
template <int R, int CO>
struct StageB {
  static constexpr int NV = R * CO / 8, P = (NV + NTC - 1) / NTC;
  static_assert(CO % 8 == 0, "a piece stays within one row");
  u32x4 r[P];
  __device__ __forceinline__ void load(const bf16 *src) {
#pragma unroll
    for (int m = 0; m < P; ++m) {
      const int e = threadIdx.x + NTC * m;
      if (NV % NTC == 0 || e < NV) r[m] = reinterpret_cast<const u32x4 *>(src)[e];
    }
  }
  __device__ __forceinline__ void store(bf16 *dst) const {
#pragma unroll
    for (int m = 0; m < P; ++m) {
      const int e = threadIdx.x + NTC * m;
      if (NV % NTC == 0 || e < NV)
        *reinterpret_cast<u32x4 *>(dst + (e / (CO / 8)) * (CO + 8) + 8 * (e % (CO / 8))) = r[m];
    }
  }
};

// ---- 2. chunk start states ------------------------------------------------
// One block per (sequence, head, 16-column slice); each chunk's W and Ke are
// staged whole in LDS, the next chunk's (and its U tile and gamma) being
// loaded into registers while this one is computed.
template <int D, int C, typename WT>
__device__ __forceinline__ void state_chain(int b, const int *__restrict__ cu, int N, int H,
                                            int seq_len, const float *__restrict__ s0,
                                            BwdLayout L, char *ws, float *sm) {
  using Sh = ChainShape<D, C>;
  constexpr int NS = Sh::NS, LD = Sh::LD, LU = Sh::LU, NRB = Sh::NRB, NCB = Sh::NCB;
  constexpr int CBW = Sh::CBW;
  float *sW = sm, *sK = sW + C * LD;          // [C][LD] row-major
  float *sSt = sK + C * LD, *sUt = sSt + 16 * LD;  // S^T [16][LD], Unew^T [16][LU]
  int slice, pair;
  if (!chain_block<NS>(b, N * H, &slice, &pair)) return;
  const int seq = pair / H, h = pair % H;
  const int col0 = slice * 16;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_rb = wv < NRB;
  int first, nch, len;
  seq_chunks(seq, cu, seq_len, C, reinterpret_cast<const int *>(ws + L.seq_first), &first,
             &nch, &len);
  if (nch == 0) return;
  // S[j][i] = S[16 cb + 4 lg + i][col0 + lr], cb = wv CBW + j
  f32x4 S[CBW];
#pragma unroll
  for (int j = 0; j < CBW; ++j) {
    const int cb = wv * CBW + j;
    S[j] = zero4();
    if (s0 && cb < NCB) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[j][i] = s0[((int64_t)pair * D + 16 * cb + 4 * lg + i) * D + col0 + lr];
    }
  }
  // one chunk's operands: W and Ke whole, the wave's U tile, e^{G_n}
  struct Buf {
    Stage<C, D, WT> w, k;
    f32x4 u, g[CBW];
  };
  auto fetch = [&](Buf &B, int ci) {  // chunk min(ci, nch - 1): always in range
    const int64_t tile = (int64_t)(first + min(ci, nch - 1)) * H + h;
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    const WT *w, *ke;
    chain_operands<WT>(L, ws, tile, C, D, &w, &ke);
    B.w.load(w);
    B.k.load(ke);
    B.u = zero4();
    if (has_rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) B.u[i] = p.u[(16 * wv + 4 * lg + i) * D + col0 + lr];
    }
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = min(wv * CBW + j, NCB - 1);
      B.g[j] = *reinterpret_cast<const f32x4 *>(p.gam + 16 * cb + 4 * lg);
    }
  };
  // Two buffers in turn: a chunk's operands are requested two steps before
  // their use, so their loads overlap two steps of products.
  auto step = [&](Buf &B, int ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    float *sc = reinterpret_cast<float *>(ws + L.sc) + tile * D * D;
    __syncthreads();  // the previous chunk is done with the LDS operands
    B.w.store(sW);
    B.k.store(sK);
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (cb < NCB) {
        *reinterpret_cast<f32x4 *>(sSt + lr * LD + 16 * cb + 4 * lg) = S[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[(16 * cb + 4 * lg + i) * D + col0 + lr] = S[j][i];
      }
    }
    const f32x4 u0 = B.u;
    f32x4 gam[CBW];
#pragma unroll
    for (int j = 0; j < CBW; ++j) gam[j] = B.g[j];
    __syncthreads();
    fetch(B, ci + 2);
    // Unew = U - W S for the wave's token block
    if (has_rb) {
      f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 16) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(sW + (16 * wv + lr) * LD + k0 + 4 * lg);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(sSt + lr * LD + k0 + 4 * lg);
        if ((k0 / 16) & 1) a1 = mma_f32_k16(a, b, a1);
        else a0 = mma_f32_k16(a, b, a0);
      }
      *reinterpret_cast<f32x4 *>(sUt + lr * LU + 16 * wv + 4 * lg) = u0 - (a0 + a1);
    }
    __syncthreads();
    // S = Diag(gam) S + Ke^T Unew for the wave's channel blocks
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (NCB % 4 == 0 || cb < NCB) {
        f32x4 acc = S[j] * gam[j];
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 16) {
          f32x4 a;
#pragma unroll
          for (int u = 0; u < 4; ++u) a[u] = sK[(k0 + 4 * lg + u) * LD + 16 * cb + lr];
          const f32x4 b = *reinterpret_cast<const f32x4 *>(sUt + lr * LU + k0 + 4 * lg);
          acc = mma_f32_k16(a, b, acc);
        }
        S[j] = acc + 0.f;  // a real VALU read of the result, before any branch
      }
    }
  };
  Buf b0, b1;
  fetch(b0, 0);
  fetch(b1, 1);
  for (int ci = 0; ci < nch; ci += 2) {
    step(b0, ci);
    if (ci + 1 < nch) step(b1, ci + 1);
  }
}

// ---- 3. state gradients, chunks in reverse ---------------------------------
template <int D, int C, typename WT>
__device__ __forceinline__ void dstate_chain(int b, const int *__restrict__ cu, int N, int H,
                                             int seq_len, const float *__restrict__ dsf,
                                             float *__restrict__ ds0, BwdLayout L, char *ws,
                                             float *sm) {
  using Sh = ChainShape<D, C>;
  constexpr int NS = Sh::NS, LD = Sh::LD, LU = Sh::LU, NRB = Sh::NRB;
  constexpr int NCB = Sh::NCB, CBW = Sh::CBW;
  float *sW = sm, *sK = sW + C * LD;               // [C][LD] row-major
  float *sDt = sK + C * LD, *sUt = sDt + 16 * LD;  // dS_next^T [16][LD], dUnew^T [16][LU]
  int slice, pair;
  if (!chain_block<NS>(b, N * H, &slice, &pair)) return;
  const int seq = pair / H, h = pair % H;
  const int col0 = slice * 16;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_rb = wv < NRB;
  int first, nch, len;
  seq_chunks(seq, cu, seq_len, C, reinterpret_cast<const int *>(ws + L.seq_first), &first,
             &nch, &len);
  // dS[j][i] = dS_next[16 cb + 4 lg + i][col0 + lr], cb = wv CBW + j
  f32x4 dS[CBW];
#pragma unroll
  for (int j = 0; j < CBW; ++j) {
    const int cb = wv * CBW + j;
    dS[j] = zero4();
    if (dsf && cb < NCB) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dS[j][i] = dsf[((int64_t)pair * D + 16 * cb + 4 * lg + i) * D + col0 + lr];
    }
  }
  // one chunk's operands: W and Ke whole, the wave's tiles of X = P^T dO
  // (its token block) and of Y = Qt^T dO (its channel blocks), e^{G_n}
  struct Buf {
    Stage<C, D, WT> w, k;
    f32x4 x, y[CBW], g[CBW];
  };
  auto fetch = [&](Buf &B, int ci) {  // chunk max(ci, 0): always in range
    const int64_t tile = (int64_t)(first + max(ci, 0)) * H + h;
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    const WT *w, *ke;
    chain_operands<WT>(L, ws, tile, C, D, &w, &ke);
    B.w.load(w);
    B.k.load(ke);
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = min(wv * CBW + j, NCB - 1);
      B.g[j] = *reinterpret_cast<const f32x4 *>(p.gam + 16 * cb + 4 * lg);
      B.y[j] = *reinterpret_cast<const f32x4 *>(p.qy + (col0 + lr) * D + 16 * cb + 4 * lg);
    }
    B.x = zero4();
    if (has_rb) B.x = *reinterpret_cast<const f32x4 *>(p.px + (col0 + lr) * C + 16 * wv + 4 * lg);
  };
  // Two buffers in turn, as in the state chain (here in reverse chunk order).
  auto step = [&](Buf &B, int ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    float *dse = reinterpret_cast<float *>(ws + L.dse) + tile * D * D;
    float *dun = reinterpret_cast<float *>(ws + L.dun) + tile * C * D;
    __syncthreads();  // the previous chunk is done with the LDS operands
    B.w.store(sW);
    B.k.store(sK);
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (cb < NCB) {
        *reinterpret_cast<f32x4 *>(sDt + lr * LD + 16 * cb + 4 * lg) = dS[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) dse[(16 * cb + 4 * lg + i) * D + col0 + lr] = dS[j][i];
      }
    }
    const f32x4 x0 = B.x;
    f32x4 gam[CBW], y0[CBW];
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      gam[j] = B.g[j];
      y0[j] = B.y[j];
    }
    __syncthreads();
    fetch(B, ci - 2);
    // dUnew = P^T dO + Ke dS_next for the wave's token block
    if (has_rb) {
      f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 16) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(sK + (16 * wv + lr) * LD + k0 + 4 * lg);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(sDt + lr * LD + k0 + 4 * lg);
        if ((k0 / 16) & 1) a1 = mma_f32_k16(a, b, a1);
        else a0 = mma_f32_k16(a, b, a0);
      }
      const f32x4 du = x0 + (a0 + a1);
      *reinterpret_cast<f32x4 *>(sUt + lr * LU + 16 * wv + 4 * lg) = du;
#pragma unroll
      for (int i = 0; i < 4; ++i) dun[(16 * wv + 4 * lg + i) * D + col0 + lr] = du[i];
    }
    __syncthreads();
    // dS = Diag(gam) dS_next + Qt^T dO - W^T dUnew for the wave's channel blocks
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (NCB % 4 == 0 || cb < NCB) {
        f32x4 aw = zero4();
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 16) {
          f32x4 wa;
#pragma unroll
          for (int u = 0; u < 4; ++u) wa[u] = sW[(k0 + 4 * lg + u) * LD + 16 * cb + lr];
          const f32x4 ub = *reinterpret_cast<const f32x4 *>(sUt + lr * LU + k0 + 4 * lg);
          aw = mma_f32_k16(wa, ub, aw);
        }
        dS[j] = dS[j] * gam[j] + (y0[j] - aw);
      }
    }
  };
  Buf b0, b1;
  if (nch > 0) {  // an empty sequence has no tiles: only dS_0 = dS_final below
    fetch(b0, nch - 1);
    fetch(b1, nch - 2);
  }
  for (int ci = nch - 1; ci >= 0; ci -= 2) {
    step(b0, ci);
    if (ci > 0) step(b1, ci - 1);
  }
  if (ds0) {
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (cb < NCB) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ds0[((int64_t)pair * D + 16 * cb + 4 * lg + i) * D + col0 + lr] = dS[j][i];
      }
    }
  }
}

// ---- 2b/3b. the two chains on the bf16 matrix cores ------------------------
// Same walks, grids and outputs as above, for bf16 inputs with C >= 32.  The
// chains stage W (or Ke) row-major and Ke^T (or W^T) as bf16, and round the
// state (or state gradient) and the Unew (or dUnew) tile to bf16 where they
// enter a product, as the forward's chain rounds its state.  The state and
// its gradient are carried in fp32; what they store per chunk for the
// gradient kernel is that bf16 rounding (16-byte row pieces from the LDS
// operand copy), and dUnew is stored in fp32.  Each product is D / 32 or
// C / 32 steps of v_mfma_f32_16x16x32_bf16 per 16 x 16 tile, where the fp32
// form needs eight times as many fp32 instructions of twice the cycles.
// Rows 0 .. R-1, columns col0 .. col0 + 15 of a row-major bf16 matrix (row
// stride ld), from their transposed copy in LDS (tr[c][r] at tr + c * ldt + r):
// two 16-byte row pieces per row, one per thread.
template <int R>
__device__ __forceinline__ void store_rows_bf16(bf16 *dst, int ld, int col0, const bf16 *tr,
                                                int ldt) {
  for (int e = threadIdx.x; e < 2 * R; e += NTC) {
    const int r = e >> 1, c8 = 8 * (e & 1);
    bf16x8 v;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = tr[(c8 + u) * ldt + r];
    *reinterpret_cast<bf16x8 *>(dst + (int64_t)r * ld + col0 + c8) = v;
  }
}

template <int D, int C>
__device__ __forceinline__ void state_chain_bf(int b, const int *__restrict__ cu, int N, int H,
                                               int seq_len, const float *__restrict__ s0,
                                               BwdLayout L, char *ws, float *sm) {
  using Sh = ChainShape<D, C>;
  constexpr int NRB = Sh::NRB, NCB = Sh::NCB, CBW = Sh::CBW;
  constexpr int LB = D + 8, LT = C + 8;
  bf16 *sW = reinterpret_cast<bf16 *>(sm), *sKT = sW + C * LB;  // [C][LB], [D][LT]
  bf16 *sSt = sKT + D * LT, *sUt = sSt + 16 * LB;                // S^T [16][LB], Unew^T [16][LT]
  int slice, pair;
  if (!chain_block<Sh::NS>(b, N * H, &slice, &pair)) return;
  const int seq = pair / H, h = pair % H;
  const int col0 = slice * 16;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_rb = wv < NRB;
  int first, nch, len;
  seq_chunks(seq, cu, seq_len, C, reinterpret_cast<const int *>(ws + L.seq_first), &first,
             &nch, &len);
  if (nch == 0) return;
  // S[j][i] = S[16 cb + 4 lg + i][col0 + lr], cb = wv CBW + j
  f32x4 S[CBW];
#pragma unroll
  for (int j = 0; j < CBW; ++j) {
    const int cb = wv * CBW + j;
    S[j] = zero4();
    if (s0 && cb < NCB) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[j][i] = s0[((int64_t)pair * D + 16 * cb + 4 * lg + i) * D + col0 + lr];
    }
  }
  struct Buf {
    StageB<C, D> w;
    StageB<D, C> k;
    f32x4 u, g[CBW];
  };
  auto fetch = [&](Buf &B, int ci) {  // chunk min(ci, nch - 1): always in range
    const int64_t tile = (int64_t)(first + min(ci, nch - 1)) * H + h;
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    const bf16 *w, *ke, *wt, *ket;
    chain_operands<bf16>(L, ws, tile, C, D, &w, &ke);
    chain_operands_t(L, ws, tile, C, D, &wt, &ket);
    B.w.load(w);
    B.k.load(ket);
    B.u = zero4();
    if (has_rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) B.u[i] = p.u[(16 * wv + 4 * lg + i) * D + col0 + lr];
    }
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = min(wv * CBW + j, NCB - 1);
      B.g[j] = *reinterpret_cast<const f32x4 *>(p.gam + 16 * cb + 4 * lg);
    }
  };
  auto step = [&](Buf &B, int ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    bf16 *sc = reinterpret_cast<bf16 *>(ws + L.sc) + tile * D * D;
    __syncthreads();  // the previous chunk is done with the LDS operands
    B.w.store(sW);
    B.k.store(sKT);
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (cb < NCB)
        *reinterpret_cast<bf16x4 *>(sSt + lr * LB + 16 * cb + 4 * lg) = to_bf16x4(S[j]);
    }
    const f32x4 u0 = B.u;
    f32x4 gam[CBW];
#pragma unroll
    for (int j = 0; j < CBW; ++j) gam[j] = B.g[j];
    __syncthreads();
    fetch(B, ci + 2);
    store_rows_bf16<D>(sc, D, col0, sSt, LB);  // the chunk's start state, as the products use it
    // Unew = U - W S for the wave's token block
    if (has_rb) {
      f32x4 a0 = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sW + (16 * wv + lr) * LB + k0 + 8 * lg);
        const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(sSt + lr * LB + k0 + 8 * lg);
        a0 = mma_k32(a, bb, a0);
      }
      *reinterpret_cast<bf16x4 *>(sUt + lr * LT + 16 * wv + 4 * lg) = to_bf16x4(u0 - a0);
    }
    __syncthreads();
    // S = Diag(gam) S + Ke^T Unew for the wave's channel blocks
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (NCB % 4 == 0 || cb < NCB) {
        f32x4 acc = S[j] * gam[j];
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8 *>(sKT + (16 * cb + lr) * LT + k0 + 8 * lg);
          const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(sUt + lr * LT + k0 + 8 * lg);
          acc = mma_k32(a, bb, acc);
        }
        S[j] = acc + 0.f;  // a real VALU read of the result, before any branch
      }
    }
  };
  Buf b0, b1;
  fetch(b0, 0);
  fetch(b1, 1);
  for (int ci = 0; ci < nch; ci += 2) {
    step(b0, ci);
    if (ci + 1 < nch) step(b1, ci + 1);
  }
}

template <int D, int C>
__device__ __forceinline__ void dstate_chain_bf(int b, const int *__restrict__ cu, int N, int H,
                                                int seq_len, const float *__restrict__ dsf,
                                                float *__restrict__ ds0, BwdLayout L, char *ws,
                                                float *sm) {
  using Sh = ChainShape<D, C>;
  constexpr int NRB = Sh::NRB, NCB = Sh::NCB, CBW = Sh::CBW;
  constexpr int LB = D + 8, LT = C + 8;
  bf16 *sK = reinterpret_cast<bf16 *>(sm), *sWT = sK + C * LB;  // [C][LB], [D][LT]
  bf16 *sDt = sWT + D * LT, *sUt = sDt + 16 * LB;  // dS_next^T [16][LB], dUnew^T [16][LT]
  int slice, pair;
  if (!chain_block<Sh::NS>(b, N * H, &slice, &pair)) return;
  const int seq = pair / H, h = pair % H;
  const int col0 = slice * 16;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool has_rb = wv < NRB;
  int first, nch, len;
  seq_chunks(seq, cu, seq_len, C, reinterpret_cast<const int *>(ws + L.seq_first), &first,
             &nch, &len);
  // dS[j][i] = dS_next[16 cb + 4 lg + i][col0 + lr], cb = wv CBW + j
  f32x4 dS[CBW];
#pragma unroll
  for (int j = 0; j < CBW; ++j) {
    const int cb = wv * CBW + j;
    dS[j] = zero4();
    if (dsf && cb < NCB) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dS[j][i] = dsf[((int64_t)pair * D + 16 * cb + 4 * lg + i) * D + col0 + lr];
    }
  }
  struct Buf {
    StageB<C, D> k;
    StageB<D, C> w;
    f32x4 x, y[CBW], g[CBW];
  };
  auto fetch = [&](Buf &B, int ci) {  // chunk max(ci, 0): always in range
    const int64_t tile = (int64_t)(first + max(ci, 0)) * H + h;
    const TilePtr p = tile_ptrs(L, ws, tile, C, D);
    const bf16 *w, *ke, *wt, *ket;
    chain_operands<bf16>(L, ws, tile, C, D, &w, &ke);
    chain_operands_t(L, ws, tile, C, D, &wt, &ket);
    B.k.load(ke);
    B.w.load(wt);
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = min(wv * CBW + j, NCB - 1);
      B.g[j] = *reinterpret_cast<const f32x4 *>(p.gam + 16 * cb + 4 * lg);
      B.y[j] = *reinterpret_cast<const f32x4 *>(p.qy + (col0 + lr) * D + 16 * cb + 4 * lg);
    }
    B.x = zero4();
    if (has_rb) B.x = *reinterpret_cast<const f32x4 *>(p.px + (col0 + lr) * C + 16 * wv + 4 * lg);
  };
  auto step = [&](Buf &B, int ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    bf16 *dse = reinterpret_cast<bf16 *>(ws + L.dse) + tile * D * D;
    float *dun = reinterpret_cast<float *>(ws + L.dun) + tile * C * D;
    __syncthreads();  // the previous chunk is done with the LDS operands
    B.k.store(sK);
    B.w.store(sWT);
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (cb < NCB)
        *reinterpret_cast<bf16x4 *>(sDt + lr * LB + 16 * cb + 4 * lg) = to_bf16x4(dS[j]);
    }
    const f32x4 x0 = B.x;
    f32x4 gam[CBW], y0[CBW];
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      gam[j] = B.g[j];
      y0[j] = B.y[j];
    }
    __syncthreads();
    fetch(B, ci - 2);
    store_rows_bf16<D>(dse, D, col0, sDt, LB);  // the state gradient after the chunk
    // dUnew = P^T dO + Ke dS_next for the wave's token block
    if (has_rb) {
      f32x4 a0 = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sK + (16 * wv + lr) * LB + k0 + 8 * lg);
        const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(sDt + lr * LB + k0 + 8 * lg);
        a0 = mma_k32(a, bb, a0);
      }
      const f32x4 du = x0 + a0;
      *reinterpret_cast<bf16x4 *>(sUt + lr * LT + 16 * wv + 4 * lg) = to_bf16x4(du);
#pragma unroll
      for (int i = 0; i < 4; ++i) dun[(16 * wv + 4 * lg + i) * D + col0 + lr] = du[i];
    }
    __syncthreads();
    // dS = Diag(gam) dS_next + Qt^T dO - W^T dUnew for the wave's channel blocks
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (NCB % 4 == 0 || cb < NCB) {
        f32x4 aw = zero4();
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8 *>(sWT + (16 * cb + lr) * LT + k0 + 8 * lg);
          const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(sUt + lr * LT + k0 + 8 * lg);
          aw = mma_k32(a, bb, aw);
        }
        dS[j] = dS[j] * gam[j] + (y0[j] - aw);
      }
    }
  };
  Buf b0, b1;
  if (nch > 0) {  // an empty sequence has no tiles: only dS_0 = dS_final below
    fetch(b0, nch - 1);
    fetch(b1, nch - 2);
  }
  for (int ci = nch - 1; ci >= 0; ci -= 2) {
    step(b0, ci);
    if (ci > 0) step(b1, ci - 1);
  }
  if (ds0) {
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (cb < NCB) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ds0[((int64_t)pair * D + 16 * cb + 4 * lg + i) * D + col0 + lr] = dS[j][i];
      }
    }
  }
}

template <int D, int C, typename WT>
__device__ __forceinline__ void run_state_chain(int b, const int *cu, int N, int H, int seq_len,
                                                const float *s0, BwdLayout L, char *ws,
                                                float *sm) {
  if constexpr (chain_bf16<C, WT>())
    state_chain_bf<D, C>(b, cu, N, H, seq_len, s0, L, ws, sm);
  else
    state_chain<D, C, WT>(b, cu, N, H, seq_len, s0, L, ws, sm);
}

template <int D, int C, typename WT>
__device__ __forceinline__ void run_dstate_chain(int b, const int *cu, int N, int H, int seq_len,
                                                 const float *dsf, float *ds0, BwdLayout L,
                                                 char *ws, float *sm) {
  if constexpr (chain_bf16<C, WT>())
    dstate_chain_bf<D, C>(b, cu, N, H, seq_len, dsf, ds0, L, ws, sm);
  else
    dstate_chain<D, C, WT>(b, cu, N, H, seq_len, dsf, ds0, L, ws, sm);
}

// ---- chain launches ----------------------------------------------------------
template <int D, int C, typename WT>
__global__ __launch_bounds__(NTC) void bwd_state_kernel(const int *__restrict__ cu, int N, int H,
                                                       int seq_len, const float *__restrict__ s0,
                                                       BwdLayout L, char *ws) {
  extern __shared__ __align__(16) float sm[];
  run_state_chain<D, C, WT>((int)blockIdx.x, cu, N, H, seq_len, s0, L, ws, sm);
}

template <int D, int C, typename WT>
__global__ __launch_bounds__(NTC) void bwd_dstate_kernel(const int *__restrict__ cu, int N, int H,
                                                        int seq_len, const float *__restrict__ dsf,
                                                        float *__restrict__ ds0, BwdLayout L,
                                                        char *ws) {
  extern __shared__ __align__(16) float sm[];
  run_dstate_chain<D, C, WT>((int)blockIdx.x, cu, N, H, seq_len, dsf, ds0, L, ws, sm);
}

// The two chains are independent: the state-gradient recursion reads W, Ke
// and the products X, Y of the per-tile pass, but never the states.  When both grids fit the GPU at once,
// one launch runs them side by side: workgroups below `split` walk the state
// gradients backward, the others the states forward.  `split` is a multiple
// of 8, so each part keeps a pair's slices on one XCD.
template <int D, int C, typename WT>
__global__ __launch_bounds__(NTC) void bwd_chains_kernel(
    const int *__restrict__ cu, int N, int H, int seq_len, const float *__restrict__ s0,
    const float *__restrict__ dsf, float *__restrict__ ds0, BwdLayout L, char *ws, int split) {
  extern __shared__ __align__(16) float sm[];
  const int b = (int)blockIdx.x;
  if (b < split)
    run_dstate_chain<D, C, WT>(b, cu, N, H, seq_len, dsf, ds0, L, ws, sm);
  else
    run_state_chain<D, C, WT>(b - split, cu, N, H, seq_len, s0, L, ws, sm);
}

// ---- 4. per-tile gradients -------------------------------------------------
// The C x C intermediates (dP, dT / dA, T^T dT) live in LDS; the C x d ones
// go through the tile's workspace scratch.  Paired products accumulate in
// registers.  The last pass forms dq, dk, dv and dbeta and, from the inputs
// q and k, the per-element dG = k (dKt e^G - dKh e^-G - dKe e^(G_n - G)) +
// q dQt e^G (= dKt Kt - dKh Kh + dQt Qt - dKe Ke), kept in LDS for the
// reverse cumulative sum that gives dg.
template <typename T, int D, int C>
__global__ __launch_bounds__((bwd_threads<D, C>())) void bwd_grad_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ d_o, const int4 *__restrict__ tab, int N, int H, int seq_len,
    T *__restrict__ dq, T *__restrict__ dk, T *__restrict__ dv, float *__restrict__ dg,
    float *__restrict__ dbeta, BwdLayout L, char *ws) {
  constexpr int NT = bwd_threads<D, C>();
  constexpr int MM = cmax(cmax(mm_lds<C, D, D>(), mm_lds<C, C, D>()),
                          cmax(mm_lds<C, D, C>(), mm_lds<C, C, C>()));
  constexpr int CC = C * C, CD = C * D;
  // dG [C][D] and the per-row-group partials of colsum(dKe Ke) [CSR][D]
  // reuse the staging and dP / dM space once the last product is done;
  // T^T dT's space then holds rowsum(dA M)
  constexpr int RT = D / 4;                                 // threads per row (last pass)
  constexpr int CSR = (NT < CD / 4 ? NT : CD / 4) / RT;     // row groups of the last pass
  static_assert(CD + CSR * D <= MM + 2 * CC, "LDS reuse at the end");
  __shared__ __align__(16) float s_big[MM + 3 * CC];
  __shared__ float s_dgam[D];
  float(&s_mm)[MM] = *reinterpret_cast<float(*)[MM]>(s_big);  // product staging
  float *s_dp = s_big + MM, *s_dt = s_dp + CC, *s_xm = s_dt + CC;
  float *s_dG = s_big, *s_cs = s_big + CD, *s_dbr = s_xm;
  const int h = (int)(blockIdx.x % (unsigned)H), c = (int)(blockIdx.x / (unsigned)H);
  const ChunkLoc loc = chunk_loc(c, tab, N, seq_len, C);
  const int t0 = loc.t0, n = loc.n;
  if (n == 0) return;
  const int64_t tile = (int64_t)c * H + h;
  const TilePtr p = tile_ptrs(L, ws, tile, C, D);
  // chunk start states and state gradients: bf16 where the chains run on
  // the bf16 matrix cores (rounded as their products use them), else fp32.
  // dUnew stays fp32: dv = Diag(beta) T^T dUnew sums it with cancellation.
  using ST = typename std::conditional<chain_bf16<C, T>(), bf16, float>::type;
  const ST *sc = reinterpret_cast<const ST *>(ws + L.sc) + tile * D * D;
  const ST *dse = reinterpret_cast<const ST *>(ws + L.dse) + tile * D * D;
  const float *dun = reinterpret_cast<const float *>(ws + L.dun) + tile * CD;
  float *x = reinterpret_cast<float *>(ws + L.scratch) + tile * L.scratch_per_tile;
  // U - W S and the staged dO feed only bf16 products for bf16 inputs, which
  // round them to bf16 as they stage them: stored in bf16 there (same bits)
  using XT = typename std::conditional<sizeof(T) == 2, bf16, float>::type;
  XT *unew = reinterpret_cast<XT *>(x), *dot = reinterpret_cast<XT *>(x + CD);
  float *dqt = x + 2 * CD, *dke = x + 3 * CD, *dw = x + 4 * CD;
  float *dbkt = x + 5 * CD, *dbv = x + 6 * CD, *dkt = x + 7 * CD, *dkh = x + 8 * CD;
  const int tid = threadIdx.x;
  const int64_t rs = (int64_t)H * D;
  for (int e4 = tid; e4 < CD / 4; e4 += NT) {
    const int r = e4 / (D / 4), i = 4 * (e4 % (D / 4));
    const float live = r < n ? 1.f : 0.f;
    const f32x4 v4 = load4_f32<T>(d_o + (int64_t)(t0 + min(r, n - 1)) * rs + (int64_t)h * D + i) * live;
    if constexpr (sizeof(T) == 2)
      *reinterpret_cast<bf16x4 *>(dot + 4 * e4) = to_bf16x4(v4);
    else
      *reinterpret_cast<f32x4 *>(dot + 4 * e4) = v4;
  }
  __syncthreads();
  block_mm_init<C, D, D, false, false, false, NT>(unew, D, p.u, -1.f, p.w, D, sc, D, s_mm);  // U - W S
  row_dots<D, D, NT>(s_dgam, dse, sc, D, false);                   // dgam = rowsum(dS_next * S)
  constexpr bool BF = sizeof(T) == 2;  // bf16 matrix cores where both operands allow
  block_mm<C, C, D, false, true, BF, NT>(s_dp, C, dot, D, unew, D, 1.f, false, s_mm);  // dO Unew^T
  for (int e = tid; e < CC; e += NT)
    if (e % C > e / C) s_dp[e] = 0.f;  // dP: lower incl. diagonal
  __syncthreads();
  // dQt = dO S^T + dP Kh and dW = -dUnew S^T; on the bf16 matrix cores one
  // staging of S serves both (the fp32 form's staging of two left operands
  // does not fit the LDS buffer)
  if constexpr (BF) {
    constexpr int TPW = MmTiles<C, D, NT>::TPW;
    f32x4 cq[TPW], cw[TPW];
#pragma unroll
    for (int q = 0; q < TPW; ++q) cq[q] = cw[q] = zero4();
    f32x4 *const cs[2] = {cq, cw};
    mm_accumulate_n<C, D, D, false, true, 2, BF, NT>(cs, dot, dun, D, sc, D, s_mm);
    mm_accumulate<C, D, C, false, false, BF, NT>(cq, s_dp, C, p.kh, D, s_mm);
    mm_store<C, D, NT>(dqt, D, static_cast<const float *>(nullptr), 1.f, cq);
    mm_store<C, D, NT>(dw, D, static_cast<const float *>(nullptr), -1.f, cw);
  } else {
    block_mm2<C, D, D, false, true, C, false, false, BF, NT>(dqt, D, dot, D, sc, D, s_dp, C, p.kh,
                                                         D, s_mm);
    block_mm<C, D, D, false, true, BF, NT>(dw, D, dun, D, sc, D, -1.f, false, s_mm);
  }
  block_mm<C, D, D, false, true, BF, NT>(dke, D, unew, D, dse, D, 1.f, false, s_mm);  // Unew dS_next^T
  // dT = (dW Kt^T + dUnew V^T) Diag(beta)
  block_mm2<C, C, D, false, true, D, false, true, BF, NT>(s_dt, C, dw, D, p.kt, D, dun, D,
                                                      reinterpret_cast<const T *>(p.vr), D,
                                                      s_mm);
  for (int e = tid; e < CC; e += NT) s_dt[e] *= p.bt[e % C];
  __syncthreads();
  block_mm<C, D, C, true, false, false, NT>(dbkt, D, p.tm, C, dw, D, 1.f, false, s_mm);   // T^T dW
  block_mm<C, D, C, true, false, false, NT>(dbv, D, p.tm, C, dun, D, 1.f, false, s_mm);   // T^T dUnew
  block_mm<C, C, C, true, false, false, NT>(s_xm, C, p.tm, C, s_dt, C, 1.f, false, s_mm);  // T^T dT
  block_mm<C, C, C, false, true, BF, NT>(s_dt, C, s_xm, C, p.tm, C, -1.f, false, s_mm);  // dA (pre-mask)
  for (int e = tid; e < CC; e += NT)
    if (e % C >= e / C) s_dt[e] = 0.f;  // dA strictly lower
  __syncthreads();
  row_dots<C, C, NT>(s_dbr, s_dt, p.mm, C, false);  // rowsum(dA * M), before dA becomes dM
  for (int e = tid; e < CC; e += NT) s_dt[e] *= p.bt[e / C];  // dM = Diag(beta) dA
  __syncthreads();
  // dKt (without Diag(beta) dBKt) = dM Kh; dKh = dM^T Kt + dP^T Qt
  block_mm<C, D, C, false, false, false, NT>(dkt, D, s_dt, C, p.kh, D, 1.f, false, s_mm);
  block_mm2<C, D, C, true, false, C, true, false, false, NT>(dkh, D, s_dt, C, p.kt, D, s_dp, C, p.qt, D,
                                                  s_mm);
  // last pass: dq, dk, dv, dbeta, dG (LDS) and colsum(dKe Ke): each thread
  // sums its channels over its rows, the row groups' partials meet in LDS and
  // are added in a fixed order, so dg is the same bits on every run
  static_assert(NT % RT == 0, "a thread keeps the same four channels on every row");
  f32x4 cs = zero4();  // this thread's share of colsum(dKe Ke)
  for (int e4 = tid; e4 < CD / 4; e4 += NT) {
    const int r = e4 / RT, i = 4 * (e4 % RT), e = 4 * e4;
    const bool live = r < n;
    const float lm = live ? 1.f : 0.f;
    const int64_t at = (int64_t)(t0 + min(r, n - 1)) * rs + (int64_t)h * D + i;
    const f32x4 qv = load4_f32<T>(q + at) * lm, kv = load4_f32<T>(k + at) * lm;
    const f32x4 vv = load4_f32<T>(v + at) * lm;
    const f32x4 G = *reinterpret_cast<const f32x4 *>(p.gc + e);
    const f32x4 Gn = *reinterpret_cast<const f32x4 *>(p.gc + (C - 1) * D + i);
    const f32x4 vqt = *reinterpret_cast<const f32x4 *>(dqt + e);
    const f32x4 vbk = *reinterpret_cast<const f32x4 *>(dbkt + e);
    const f32x4 vkh = *reinterpret_cast<const f32x4 *>(dkh + e);
    const f32x4 vke = *reinterpret_cast<const f32x4 *>(dke + e);
    const f32x4 vbv = *reinterpret_cast<const f32x4 *>(dbv + e);
    const float b = p.bt[r];
    const f32x4 vkt = *reinterpret_cast<const f32x4 *>(dkt + e) + b * vbk;
    f32x4 oq, ok, dG;
    float rowp = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float eg = __expf(G[u]), emg = __expf(-G[u]), egn = __expf(Gn[u] - G[u]);
      const float tk = vkt[u] * eg, th = vkh[u] * emg, te = vke[u] * egn;
      oq[u] = vqt[u] * eg;
      ok[u] = tk + th + te;
      dG[u] = kv[u] * (tk - th - te) + qv[u] * oq[u];
      rowp += vbk[u] * kv[u] * eg + vbv[u] * vv[u];  // (dBKt * Kt) + (dBV * V)
      cs[u] += te * kv[u];                           // dKe * Ke, summed over rows
    }
    rowp = group_sum<RT>(rowp);
    if (live) {
      store4_f32<T>(dq + at, oq);
      store4_f32<T>(dk + at, ok);
      store4_f32<T>(dv + at, vbv * b);
      *reinterpret_cast<f32x4 *>(s_dG + e) = dG;
      if (e4 % RT == 0) dbeta[(int64_t)(t0 + r) * H + h] = s_dbr[r] + rowp;
    }
  }
  if (tid < CD / 4)
    *reinterpret_cast<f32x4 *>(s_cs + (tid / RT) * D + 4 * (tid % RT)) = cs;
  __syncthreads();
  // dg: reverse cumulative sum of dG over the chunk plus dG_n, per channel
  for (int i = tid; i < D; i += NT) {
    float csum = 0.f;
    for (int g = 0; g < CSR; ++g) csum += s_cs[g * D + i];
    float run = s_dgam[i] * p.gam[i] + csum;
    for (int r = n - 1; r >= 0; --r) {
      run += s_dG[r * D + i];
      dg[(int64_t)(t0 + r) * rs + (int64_t)h * D + i] = run;
    }
  }
}

template <typename T, int D, int C>
static hipError_t launch_bwd_dc(const BwdArgs &a) {
  const unsigned tiles = (unsigned)(a.grid_chunks * a.num_heads);
  const unsigned slices = chain_grid(a.num_seqs * a.num_heads, D / 16);
  const T *q = reinterpret_cast<const T *>(a.q), *k = reinterpret_cast<const T *>(a.k);
  const T *v = reinterpret_cast<const T *>(a.v), *d_o = reinterpret_cast<const T *>(a.d_o);
  constexpr size_t lds_state = state_lds_bytes<D, C, T>(), lds_dstate = dstate_lds_bytes<D, C, T>();
  constexpr size_t lds_chains = lds_state > lds_dstate ? lds_state : lds_dstate;
  // 80,384 bytes at the largest shape (d = 128, C = 64)
  static std::atomic<unsigned long long> raised1{0}, raised2{0}, raised3{0};
  hipError_t e = raise_lds_limit((const void *)bwd_state_kernel<D, C, T>, (int)lds_state, raised1);
  if (e == hipSuccess)
    e = raise_lds_limit((const void *)bwd_dstate_kernel<D, C, T>, (int)lds_dstate, raised2);
  if (e == hipSuccess)
    e = raise_lds_limit((const void *)bwd_chains_kernel<D, C, T>, (int)lds_chains, raised3);
  if (e != hipSuccess) return e;
  if (tiles > 0)
    hipLaunchKernelGGL((bwd_prep_kernel<T, D, C>), dim3(tiles), dim3(bwd_threads<D, C>()), 0, a.stream, q, k, v,
                       d_o, a.g, a.beta, a.chunk_tab, a.num_seqs, a.num_heads, a.seq_len,
                       a.lay, a.ws);
  const int cus = device_cus();
  if (cus > 0 && 2 * slices <= (unsigned)cus) {
    hipLaunchKernelGGL((bwd_chains_kernel<D, C, T>), dim3(2 * slices), dim3(NTC), lds_chains,
                       a.stream, a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len, a.s0, a.dsf,
                       a.ds0, a.lay, a.ws, (int)slices);
  } else {
    hipLaunchKernelGGL((bwd_state_kernel<D, C, T>), dim3(slices), dim3(NTC), lds_state, a.stream,
                       a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len, a.s0, a.lay, a.ws);
    hipLaunchKernelGGL((bwd_dstate_kernel<D, C, T>), dim3(slices), dim3(NTC), lds_dstate, a.stream,
                       a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len, a.dsf, a.ds0, a.lay,
                       a.ws);
  }
  if (tiles > 0)
    hipLaunchKernelGGL((bwd_grad_kernel<T, D, C>), dim3(tiles), dim3(bwd_threads<D, C>()), 0, a.stream, q, k,
                       v, d_o, a.chunk_tab, a.num_seqs, a.num_heads, a.seq_len,
                       reinterpret_cast<T *>(a.dq), reinterpret_cast<T *>(a.dk),
                       reinterpret_cast<T *>(a.dv), a.dg, a.dbeta, a.lay, a.ws);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_bwd_d(const BwdArgs &a) {
  switch (a.chunk) {
    case 16: return launch_bwd_dc<T, D, 16>(a);
    case 32: return launch_bwd_dc<T, D, 32>(a);
    case 64: return launch_bwd_dc<T, D, 64>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs &a, kda_dtype dt) {
  if (a.grid_chunks == 0 && a.ds0 == nullptr) return hipSuccess;
  if (dt == KDA_DTYPE_BF16) {
    switch (a.d) {
      case 32: return launch_bwd_d<bf16, 32>(a);
      case 64: return launch_bwd_d<bf16, 64>(a);
      case 128: return launch_bwd_d<bf16, 128>(a);
    }
  } else {
    switch (a.d) {
      case 32: return launch_bwd_d<float, 32>(a);
      case 64: return launch_bwd_d<float, 64>(a);
      case 128: return launch_bwd_d<float, 128>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
