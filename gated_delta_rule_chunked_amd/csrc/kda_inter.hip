// kda_inter.hip -- inter-chunk kernel: carries the state from chunk to chunk.
//
// Between chunks the state is propagated sequentially; inside a chunk the
// intra-chunk factors turn the token updates into dense products
// (mkdocs.reaper.mx "Attention lineaire et recurrence", section "Le calcul
// par blocs": sequential between blocks, parallel inside; fr.news.hada.io
// Kimi Linear summary, section "Algorithme parallele par chunks": the final
// state of a chunk is the initial state of the next, the state update is in
// matrix form, the output combines the inter-chunk recurrent part and the
// intra-chunk parallel part).  For a chunk entering with state S:
//
//   Unew = U - W S                       (the per-token delta-rule updates)
//   O    = Qt S + P Unew                 (read-out after each token's update)
//   S   <- Diag(e^{G_n}) S + Ke^T Unew   (state after the chunk)
//
// Every product multiplies S from the left, so the d_v columns of S evolve
// independently: a workgroup owns one (sequence, head, column slice of width
// BV) and runs over that sequence's chunks.  The fp32 state slice lives in
// registers (distributed as 16x16 matrix-core output tiles over the four
// wavefronts) and is mirrored in LDS in the operand type for the next
// chunk's products; Unew passes through LDS once per chunk.  Two barriers
// per chunk.  Workgroups of the same (sequence, head) are placed on the same
// XCD so that their shared reads of W, Qt, P and Ke hit one L2.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <typename T, int D, int C, int BV>
struct InterCfg {
  static constexpr int NRB = C / 16;       // 16-token blocks of a chunk
  static constexpr int NSRB = D / 16;      // 16-channel blocks of the state
  static constexpr int NCBV = BV / 16;     // 16-column blocks of the slice
  static constexpr int CK = C < 32 ? 32 : C;
  static constexpr int PAD = 16 / (int)sizeof(T);
  static constexpr int LDS_S = D + PAD;    // sST [BV][LDS_S]  (S transposed)
  static constexpr int LDU = CK + PAD;     // sUnT [BV][LDU]   (Unew transposed)
  static constexpr int NUJ = (NRB + 3) / 4;
  static constexpr int NSJ = (NSRB + 3) / 4;
  static_assert(D % BV == 0 && BV % 16 == 0, "slice shape");
};

template <typename T, int D, int C, int BV>
__global__ __launch_bounds__(256) void inter_chunk_kernel(
    const T *__restrict__ qt, const T *__restrict__ w, const T *__restrict__ ut,
    const T *__restrict__ ket, const T *__restrict__ pm,
    const float *__restrict__ gc, const int *__restrict__ cu,
    const int *__restrict__ seq_first, int N, int H, int seq_len,
    const float *__restrict__ s0, float *__restrict__ s_final,
    T *__restrict__ o) {
  using Cfg = InterCfg<T, D, C, BV>;
  constexpr int NRB = Cfg::NRB, NSRB = Cfg::NSRB, NCBV = Cfg::NCBV, CK = Cfg::CK;
  constexpr int LDS_S = Cfg::LDS_S, LDU = Cfg::LDU, NUJ = Cfg::NUJ, NSJ = Cfg::NSJ;
  constexpr int NS = D / BV;

  __shared__ __align__(16) T sST[BV * LDS_S];
  __shared__ __align__(16) T sUnT[BV * LDU];

  // XCD-aware placement: consecutive workgroup ids go to different XCDs, so
  // the NS slices of one (sequence, head) get ids that share id % 8.
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int slice = local % NS, unit = local / NS;
  const int pair = unit * 8 + xcd;
  if (pair >= N * H) return;
  const int seq = pair / H, h = pair % H;
  int t0, t1;
  if (cu) {
    t0 = cu[seq];
    t1 = cu[seq + 1];
  } else {
    t0 = seq * seq_len;
    t1 = t0 + seq_len;
  }
  const int len = t1 - t0;
  const int nch = (len + C - 1) / C;
  const int first = nch == 0 ? 0 : (cu ? seq_first[seq] : seq * ((seq_len + C - 1) / C));

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int col0 = slice * BV;
  const int64_t rs = (int64_t)H * D;

  // ---- initial state slice into registers and LDS ----
  f32x4 S[NSJ][NCBV];
  const int64_t sbase = (int64_t)pair * D * D;
#pragma unroll
  for (int j = 0; j < NSJ; ++j) {
    const int srb = wave + 4 * j;
#pragma unroll
    for (int cb = 0; cb < NCBV; ++cb) {
      f32x4 x = zero4();
      if (srb < NSRB && s0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[i] = s0[sbase + (int64_t)(16 * srb + 4 * lg + i) * D + col0 + 16 * cb + lr];
      }
      S[j][cb] = x;
      if (srb < NSRB) store4_f32<T>(sST + (16 * cb + lr) * LDS_S + 16 * srb + 4 * lg, x);
    }
  }
  if (CK > C) {
    for (int e = tid; e < BV * (CK - C); e += 256)
      sUnT[(e / (CK - C)) * LDU + C + e % (CK - C)] = from_f32<T>(0.f);
  }
  __syncthreads();

  for (int ci = 0; ci < nch; ++ci) {
    const int64_t tile = (int64_t)(first + ci) * H + h;
    const int tc = t0 + ci * C;
    const int rows = min(C, len - ci * C);
    const T *w_t = w + tile * (C * D);
    const T *q_t = qt + tile * (C * D);
    const T *u_t = ut + tile * (D * C);
    const T *k_t = ket + tile * (D * CK);
    const T *p_t = pm + tile * (C * CK);

    // (a) Unew = U - W S and O = Qt S for this wave's token blocks
    f32x4 accO[NUJ][NCBV];
#pragma unroll
    for (int j = 0; j < NUJ; ++j) {
      const int rb = wave + 4 * j;
#pragma unroll
      for (int cb = 0; cb < NCBV; ++cb) accO[j][cb] = zero4();
      if (rb >= NRB) continue;
      typename Frag<T>::type aw[D / 32], aq[D / 32];
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        aw[ks] = load8<T>(w_t + (16 * rb + lr) * D + 32 * ks + 8 * lg);
        aq[ks] = load8<T>(q_t + (16 * rb + lr) * D + 32 * ks + 8 * lg);
      }
#pragma unroll
      for (int cb = 0; cb < NCBV; ++cb) {
        f32x4 ws = zero4(), acco = zero4();
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const auto bs = load8<T>(sST + (16 * cb + lr) * LDS_S + 32 * ks + 8 * lg);
          ws = mma_k32(aw[ks], bs, ws);
          acco = mma_k32(aq[ks], bs, acco);
        }
        const f32x4 u = load4_f32<T>(u_t + (col0 + 16 * cb + lr) * C + 16 * rb + 4 * lg);
        store4_f32<T>(sUnT + (16 * cb + lr) * LDU + 16 * rb + 4 * lg, u - ws);
        accO[j][cb] = acco;
      }
    }
    __syncthreads();

    // (c) O += P Unew, store the output rows of this wave
#pragma unroll
    for (int j = 0; j < NUJ; ++j) {
      const int rb = wave + 4 * j;
      if (rb >= NRB) continue;
#pragma unroll
      for (int cb = 0; cb < NCBV; ++cb) {
        f32x4 acco = accO[j][cb];
#pragma unroll
        for (int ks = 0; ks < CK / 32; ++ks) {
          if (32 * ks > 16 * rb + 15) break;  // P is lower triangular
          const auto ap = load8<T>(p_t + (16 * rb + lr) * CK + 32 * ks + 8 * lg);
          const auto bu = load8<T>(sUnT + (16 * cb + lr) * LDU + 32 * ks + 8 * lg);
          acco = mma_k32(ap, bu, acco);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rb + 4 * lg + i;
          if (r < rows)
            o[(int64_t)(tc + r) * rs + (int64_t)h * D + col0 + 16 * cb + lr] = from_f32<T>(acco[i]);
        }
      }
    }

    // (d) S <- Diag(e^{G_n}) S + Ke^T Unew
    const float *g_last = gc + (int64_t)(tc + rows - 1) * rs + (int64_t)h * D;
#pragma unroll
    for (int j = 0; j < NSJ; ++j) {
      const int srb = wave + 4 * j;
      if (srb >= NSRB) continue;
      const f32x4 gl = *reinterpret_cast<const f32x4 *>(g_last + 16 * srb + 4 * lg);
      const f32x4 gam = f32x4{__expf(gl[0]), __expf(gl[1]), __expf(gl[2]), __expf(gl[3])};
      typename Frag<T>::type ak[CK / 32];
#pragma unroll
      for (int ks = 0; ks < CK / 32; ++ks)
        ak[ks] = load8<T>(k_t + (16 * srb + lr) * CK + 32 * ks + 8 * lg);
#pragma unroll
      for (int cb = 0; cb < NCBV; ++cb) {
        f32x4 acc = S[j][cb] * gam;
#pragma unroll
        for (int ks = 0; ks < CK / 32; ++ks) {
          const auto bu = load8<T>(sUnT + (16 * cb + lr) * LDU + 32 * ks + 8 * lg);
          acc = mma_k32(ak[ks], bu, acc);
        }
        S[j][cb] = acc;
        store4_f32<T>(sST + (16 * cb + lr) * LDS_S + 16 * srb + 4 * lg, acc);
      }
    }
    __syncthreads();
  }

  if (s_final) {
#pragma unroll
    for (int j = 0; j < NSJ; ++j) {
      const int srb = wave + 4 * j;
      if (srb >= NSRB) continue;
#pragma unroll
      for (int cb = 0; cb < NCBV; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_final[sbase + (int64_t)(16 * srb + 4 * lg + i) * D + col0 + 16 * cb + lr] = S[j][cb][i];
    }
  }
}

template <typename T, int D, int C, int BV>
static hipError_t launch_inter_t(const FwdArgs &a) {
  constexpr int NS = D / BV;
  const int pairs = a.num_seqs * a.num_heads;
  const int units = (pairs + 7) / 8;
  const dim3 grid((unsigned)(8 * units * NS));
  char *ws = a.ws;
  hipLaunchKernelGGL((inter_chunk_kernel<T, D, C, BV>), grid, dim3(256), 0, a.stream,
                     reinterpret_cast<const T *>(ws + a.lay.qt),
                     reinterpret_cast<const T *>(ws + a.lay.w),
                     reinterpret_cast<const T *>(ws + a.lay.ut),
                     reinterpret_cast<const T *>(ws + a.lay.ket),
                     reinterpret_cast<const T *>(ws + a.lay.p),
                     reinterpret_cast<const float *>(ws + a.lay.gc), a.cu_seqlens,
                     reinterpret_cast<const int *>(ws + a.lay.seq_first), a.num_seqs,
                     a.num_heads, a.seq_len, a.s0, a.s_final, reinterpret_cast<T *>(a.o));
  return hipGetLastError();
}

// Column-slice width: narrow slices when few (sequence, head) pairs exist so
// that the launch still spreads over the compute units.
template <typename T, int D, int C>
static hipError_t launch_inter_c(const FwdArgs &a) {
  const int pairs = a.num_seqs * a.num_heads;
  if (pairs * (D / 16) <= 2048) return launch_inter_t<T, D, C, 16>(a);
  return launch_inter_t<T, D, C, 32>(a);
}

template <typename T, int D>
static hipError_t launch_inter_d(const FwdArgs &a) {
  switch (a.chunk) {
    case 16: return launch_inter_c<T, D, 16>(a);
    case 32: return launch_inter_c<T, D, 32>(a);
    case 64: return launch_inter_c<T, D, 64>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_inter(const FwdArgs &a, kda_dtype dt) {
  if (dt == KDA_DTYPE_BF16) {
    switch (a.d) {
      case 32: return launch_inter_d<bf16, 32>(a);
      case 64: return launch_inter_d<bf16, 64>(a);
      case 128: return launch_inter_d<bf16, 128>(a);
    }
  } else {
    switch (a.d) {
      case 32: return launch_inter_d<float, 32>(a);
      case 64: return launch_inter_d<float, 64>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
