// kda_intra.hip -- per-chunk kernel: chunk location, chunk-local cumulative
// log-decay, decay-scaled blocks, UT transform and WY factors for one
// (chunk, head) tile.
//
// For a chunk of n <= C tokens the token-by-token delta updates are packed
// into dense factors (fr.news.hada.io Kimi Linear summary, section
// "Algorithme parallele par chunks": WY representation, UT transform,
// row-by-row forward substitution, intra-chunk work on the matrix units;
// section "Un volume de calcul reduit": both low-rank vectors are tied to k,
// so only two chunk matrices are needed).  With G_r = g_1 + ... + g_r the
// chunk-local cumulative log-decay of every key channel (mkdocs.reaper.mx
// "Attention lineaire et recurrence", section "Le piege numerique de la
// decroissance cumulee"; it restarts at every chunk and sequence start):
//
//   Qt = Q * e^G,  Kt = K * e^G,  Kh = K * e^-G,  Ke = K * e^(G_n - G)
//   A  = strictly_lower(Diag(beta) Kt Kh^T)       (decay-scaled K K^T)
//   P  = lower_with_diagonal(Qt Kh^T)             (decay-scaled Q K^T)
//   T  = (I + A)^-1                               (forward substitution)
//   W  = T Diag(beta) Kt,   U = T Diag(beta) V    (WY factors)
//
// (* = per-channel product.)  The inter-chunk kernel then uses U - W S,
// Qt S + P (U - W S) and e^(G_n) S + Ke^T (U - W S).  The chunk-start
// reference of Kh needs G_n >= -80 per channel (e^80 is far inside fp32 and
// bf16 range), the bound quoted in the same section of mkdocs.reaper.mx for
// a 16-token tile.  A chunk that decays further in some channel takes a
// second form of A and P (tile-uniform branch): each 16-token block b is
// referenced to R_b, the cumulative decay before it, so that
//   A[i][j] = beta_i sum_e (K_i e^(G_i - R_bi)) e^(R_bi - R_bj) (K_j e^(R_bj - G_j))
// with the first two factors <= 1 and the third bounded by the decay inside
// block bj; P likewise with Q.  The bound then applies to 16-token blocks
// only; Ke takes e^(G_n - G) directly.
//
// One workgroup of 4 wavefronts per tile:
//  1. Thread t owns 4 channels x RPT consecutive tokens.  It loads its g
//     rows, then q, k, v and beta (coalesced along channels), sums g down its
//     tokens, adds the totals of the token groups above it (LDS), forms the
//     scaled rows in fp32 and stages Kt, Kh, Qt row-major in LDS; Ke,
//     Diag(beta) Kt and Diag(beta) V stay in registers.
//  2. Qt leaves LDS for the workspace.  A and P^T tiles on the matrix cores
//     (K = d); A (masked, beta-scaled) goes to LDS in fp32, P is produced as
//     P^T tiles so that each lane stores 4 consecutive positions of one P row.
//  3. Diag(beta) Kt, Diag(beta) V and Ke are staged transposed (each thread
//     writes its token run of a channel at once); T = (I + A)^-1 in fp32 LDS:
//     16 x 16 diagonal blocks by forward substitution, then the blocks below
//     them on fp32 matrix cores, one block column per wave.
//  4. Ke^T leaves LDS for the workspace.  W^T = (Diag(beta) Kt)^T T^T and
//     U = T Diag(beta) V on the matrix cores,
//     T rounded to the operand type; each wave reuses its T fragments for
//     all of its tiles.
// Every workspace tensor is written in the fragment-major, kperm-ordered
// layout the inter-chunk kernel loads (kda_common.hpp), together with
// exp(G_n) per channel.
#include <type_traits>

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

template <typename T, int D, int C>
struct IntraCfg {
  // 4 wavefronts; two workgroups fit a CU (LDS bound).  8-wavefront
  // workgroups, with half the rows per thread, measured slower on MI355X.
  static constexpr int NT = 256;
  static constexpr int NW = NT / 64;               // wavefronts per workgroup
  static constexpr int NRB = C / 16;               // 16-token blocks of the chunk
  static constexpr int NCB = D / 16;               // 16-channel blocks of a head
  static constexpr int CK = C < 32 ? 32 : C;       // token extent per K-step
  static constexpr int NKB = CK / 16;              // token blocks incl. padding
  static constexpr int KD = D / 32;                // K-steps over channels
  static constexpr int KC = CK / 32;               // K-steps over tokens
  static constexpr int CG = D / 4;                 // 4-channel groups (phase 1)
  static constexpr int RG = NT / CG;               // token groups (phase 1)
  static constexpr int RPT = (C + RG - 1) / RG;    // tokens per thread (phase 1)
  static constexpr int PAD = 16 / (int)sizeof(T);  // 16-byte row padding
  static constexpr int LDR = D + PAD;              // row-major [C][D] stride
  static constexpr int LDT = CK + PAD;             // transposed [D][CK] stride
  static constexpr int LDA = CK + 4;               // fp32 [C][CK] stride
  static constexpr int BYTES_ROW = C * LDR * (int)sizeof(T);
  static constexpr int BYTES_TR = D * LDT * (int)sizeof(T);
  static constexpr int BYTES_X = (BYTES_ROW > BYTES_TR ? BYTES_ROW : BYTES_TR) * 3;
  static constexpr int BYTES_A = C * LDA * 4;
  static constexpr int BYTES_TOT = RG * CG * 16;   // phase-1 token-group totals (alias A)
  static constexpr int BYTES_Y = BYTES_A > BYTES_TOT ? BYTES_A : BYTES_TOT;
  static constexpr int BYTES_REF = NRB * D * 4;     // per-block decay references
  static constexpr int LDS_BYTES = BYTES_X + BYTES_Y + C * 4 + BYTES_REF;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(C % 16 == 0 && D % 32 == 0 && RPT * RG >= C, "tile shape");
  static_assert(RPT == 1 || RPT == 2 || RPT % 4 == 0, "token runs per thread");
  static constexpr int NP = NRB * (NKB / 2);       // phase-2 (token block, key-block pair)
  static constexpr int NQB = NRB * KD;             // 16 x 32 fragment blocks of Qt
  static constexpr int NEB = NCB * KC;             // 16 x 32 fragment blocks of Ke^T
  // phase 4: NW / NRB waves share a token block, CPW channel blocks each
  static constexpr int WPR = NW / NRB;
  static constexpr int CPW = (NCB + WPR - 1) / WPR;
  static_assert(NW % NRB == 0, "phase-4 wave split");
};

// One lane's run of a fragment-major block: the 8 kperm positions 8 g .. 8 g + 7
// of a 32-group hold indices 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3, so
// the run is two quads of a row-major LDS row, written as 8 consecutive
// elements; a wavefront writes one contiguous 16 x 32 block.
template <typename T>
__device__ __forceinline__ void copy_run(T *dst, const T *row32) {
  *reinterpret_cast<typename Frag<T>::type *>(dst) = join4(load4<T>(row32), load4<T>(row32 + 16));
}

// A thread's run of L consecutive elements of one channel (L = 1, 2, 4, 8
// tokens), kept as one vector so that 16-bit elements share registers in
// pairs, and stored to LDS in one piece (the destination is aligned to it).
template <typename T, int L>
struct Run {
  typedef T type __attribute__((ext_vector_type(L < 2 ? 2 : L)));
};
template <typename T, int L>
__device__ __forceinline__ void store_run(T *p, const typename Run<T, L>::type &x) {
  if constexpr (L == 1)
    *p = x[0];
  else
    *reinterpret_cast<typename Run<T, L>::type *>(p) = x;
}

// RAW: the gate input is z in the operand type and in.gate selects the gate
// function; otherwise it is g itself in fp32.
template <typename T, int D, int C, bool RAW>
__global__ __launch_bounds__((IntraCfg<T, D, C>::NT)) void intra_chunk_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const void *__restrict__ gate, const float *__restrict__ beta, const OptArgs in,
    const int4 *__restrict__ tab, int N, int H, int seq_len,
    T *__restrict__ qt_out, T *__restrict__ w_out, T *__restrict__ ut_out,
    T *__restrict__ ket_out, T *__restrict__ p_out, float *__restrict__ gam_out) {
  using Cfg = IntraCfg<T, D, C>;
  using F = typename Frag<T>::type;
  constexpr int NT = Cfg::NT, NW = Cfg::NW;
  constexpr int NRB = Cfg::NRB, NCB = Cfg::NCB, CK = Cfg::CK, NKB = Cfg::NKB;
  constexpr int KD = Cfg::KD, KC = Cfg::KC, CG = Cfg::CG, RG = Cfg::RG, RPT = Cfg::RPT;
  constexpr int LDR = Cfg::LDR, LDT = Cfg::LDT, LDA = Cfg::LDA;

  extern __shared__ __align__(16) char smem[];
  T *sKt = reinterpret_cast<T *>(smem);                          // [C][LDR]
  T *sKh = reinterpret_cast<T *>(smem + Cfg::BYTES_ROW);         // [C][LDR]
  T *sQt = reinterpret_cast<T *>(smem + 2 * Cfg::BYTES_ROW);     // [C][LDR]
  T *sBKt = reinterpret_cast<T *>(smem);                         // [D][LDT] (phase 3+)
  T *sBVt = reinterpret_cast<T *>(smem + Cfg::BYTES_TR);         // [D][LDT] (phase 3+)
  T *sKeT = reinterpret_cast<T *>(smem + 2 * Cfg::BYTES_TR);     // [D][LDT] (phase 3+)
  float *sA = reinterpret_cast<float *>(smem + Cfg::BYTES_X);    // [C][LDA] (phase 2+)
  f32x4 *sTot = reinterpret_cast<f32x4 *>(smem + Cfg::BYTES_X);  // [RG][CG] (phase 1)
  float *sBeta = reinterpret_cast<float *>(smem + Cfg::BYTES_X + Cfg::BYTES_Y);
  float *sRef = reinterpret_cast<float *>(smem + Cfg::BYTES_X + Cfg::BYTES_Y + C * 4);  // [NRB][D]

  // heads vary fastest over the grid: the tiles resident together then read
  // whole token rows of the [T, H, d] inputs instead of one head's slice
  if (inputs_rejected(in)) return;
  const int h = (int)(blockIdx.x % (unsigned)H), c = (int)(blockIdx.x / (unsigned)H);
  const ChunkLoc loc = chunk_loc(c, tab, N, seq_len, C);
  const int t0 = loc.t0, n = loc.n;
  if (n == 0) return;
  const int64_t tile = (int64_t)c * H + h;
  const int tid = threadIdx.x, lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t rs = (int64_t)H * D;  // token stride of [T, H, D] tensors
  const int64_t base = (int64_t)t0 * rs + (int64_t)h * D;

  // ---------------- phase 1: cumulative decay and scaled rows ---------------
  // Every load of the phase is issued up front and unconditionally (rows past
  // the chunk end re-read its last row and are masked to zero afterwards), so
  // a thread waits for one memory round trip instead of one per row.  The
  // tile's base addresses are wavefront-uniform; per-row offsets are 32-bit
  // byte offsets (a tile spans at most 64 rows of H * d <= 2^23 elements).
  const int cg = tid % CG, rg = tid / CG;
  const int ch0 = 4 * cg, r0 = rg * RPT;
  constexpr unsigned GSZ = RAW ? (unsigned)sizeof(T) : 4u;  // bytes per gate element
  const char *gb = reinterpret_cast<const char *>(gate) + base * GSZ;
  const char *qb = reinterpret_cast<const char *>(q + base);
  const char *kb = reinterpret_cast<const char *>(k + base);
  const char *vb = reinterpret_cast<const char *>(v + base);
  const char *bb = reinterpret_cast<const char *>(beta + ((int64_t)t0 * H + h));
  f32x4 Gv[RPT];
  typename Vec4<T>::type qr[RPT], kr[RPT], vr[RPT], zr[RAW ? RPT : 1];
  float brr[RPT];
  // The gate rows go first: the cumulative sum and its LDS exchange need
  // only them, and the wait counter counts loads in issue order, so they run
  // while q, k, v and beta are still arriving (the compiler otherwise issues
  // most gate loads last; measured 6% off the kernel on long sequences).
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const unsigned r = (unsigned)min(r0 + j, n - 1);
    const unsigned off = r * (unsigned)rs + (unsigned)ch0;
    if constexpr (RAW)
      zr[j] = *reinterpret_cast<const typename Vec4<T>::type *>(gb + off * GSZ);
    else
      Gv[j] = *reinterpret_cast<const f32x4 *>(gb + off * GSZ);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const unsigned r = (unsigned)min(r0 + j, n - 1);
    const unsigned off = r * (unsigned)rs + (unsigned)ch0;
    qr[j] = *reinterpret_cast<const typename Vec4<T>::type *>(qb + off * (unsigned)sizeof(T));
    kr[j] = *reinterpret_cast<const typename Vec4<T>::type *>(kb + off * (unsigned)sizeof(T));
    vr[j] = *reinterpret_cast<const typename Vec4<T>::type *>(vb + off * (unsigned)sizeof(T));
    brr[j] = *reinterpret_cast<const float *>(bb + r * (unsigned)H * 4u);
  }

  if constexpr (RAW) {  // the gate function, in fp32
    if (in.gate == KDA_GATE_SOFTPLUS) {
      const float eA = __expf(in.gate_A[h]);
#pragma unroll
      for (int j = 0; j < RPT; ++j) Gv[j] = gate_softplus(to_f32x4(zr[j]), eA);
    } else {
#pragma unroll
      for (int j = 0; j < RPT; ++j) Gv[j] = gate_sigmoid(to_f32x4(zr[j]), in.gate_min);
    }
  }

  // Per channel of this thread's token run: Diag(beta) Kt, Diag(beta) V and
  // Ke, staged transposed in phase 3.
  typename Run<T, RPT>::type bk[4], bv[4], ke[4];
  T *qt_tile = qt_out + tile * (C * D);
  // Whether some channel of the chunk decays by more than the bound of the
  // chunk-start reference (uniform over the workgroup).
  bool far = false;
  f32x4 far_pre = zero4(), far_tot = zero4();
  // Full chunks (every tile but a sequence's last) skip the row masks.
  auto scaled_rows = [&](auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    {
      f32x4 run = zero4();
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        // row slots past the chunk (when RG * RPT > C) or past its end add nothing
        const bool in = TAIL ? r0 + j < n : (RG * RPT == C || r0 + j < C);
        run += in ? Gv[j] : zero4();
        Gv[j] = run;
      }
      sTot[rg * CG + cg] = run;
    }
    __syncthreads();
    f32x4 pre = zero4(), tot = zero4();
#pragma unroll 4
    for (int i = 0; i < RG; ++i) {
      const f32x4 x = sTot[i * CG + cg];
      if (i < rg) pre += x;
      tot += x;
    }
    const f32x4 etot = {__expf(tot[0]), __expf(tot[1]), __expf(tot[2]), __expf(tot[3])};
    if (rg == 0) *reinterpret_cast<f32x4 *>(gam_out + tile * D + ch0) = etot;
    // The chunk-start reference holds while the summed log-decay is >= -80
    // in every channel (e^80 is finite in fp32 and bf16).  Every wavefront's
    // 64 threads cover all CG channel groups (CG <= 64 divides 64) and read
    // the same totals from LDS, so a wavefront vote gives every wave the same
    // answer without a workgroup barrier.
    static_assert(64 % CG == 0, "each wavefront covers every channel group");
    far = __any(tot[0] < -80.f || tot[1] < -80.f || tot[2] < -80.f || tot[3] < -80.f) != 0;
    if (__builtin_expect(far, 0)) {  // the block-referenced rows are formed by far_rows
      far_pre = pre;
      far_tot = tot;
      return;
    }
    // e^-G = 1 / e^G and e^(G_n - G) = e^G_n / e^G: in range for G >= -80
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = r0 + j;
      if (r < C) {
        const bool live = !TAIL || r < n;
        f32x4 qv = live ? to_f32x4(qr[j]) : zero4();
        f32x4 kv = live ? to_f32x4(kr[j]) : zero4();
        const f32x4 vv = live ? to_f32x4(vr[j]) : zero4();
        if (in.l2norm_qk) {  // the CG lanes of this row hold its d channels
          qv *= l2_inv_norm<CG>(qv);
          kv *= l2_inv_norm<CG>(kv);
        }
        const float br = live ? (in.beta_logits ? sigmoid(brr[j]) : brr[j]) : 0.f;
        if (cg == 0) sBeta[r] = br;
        const f32x4 G = Gv[j] + pre;
        f32x4 qt, kt, kh;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float eg = __expf(G[e]);
          const float ei = __builtin_amdgcn_rcpf(eg);
          qt[e] = qv[e] * eg;
          kt[e] = kv[e] * eg;
          kh[e] = kv[e] * ei;
          ke[e][j] = from_f32<T>(kv[e] * (ei * etot[e]));
          bk[e][j] = from_f32<T>(br * kt[e]);
          bv[e][j] = from_f32<T>(br * vv[e]);
        }
        store4_f32<T>(sKt + r * LDR + ch0, kt);
        store4_f32<T>(sKh + r * LDR + ch0, kh);
        store4_f32<T>(sQt + r * LDR + ch0, qt);
      }
    }
  };
  // Block-referenced rows of a chunk past the bound (rare: one masked form).
  auto far_rows = [&](const f32x4 pre, const f32x4 tot) {
    constexpr bool TAIL = true;
    // R_b = G of the row before block b (0 for block 0), written by the
    // thread that owns that row
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = r0 + j;
      if (r < C - 1 && (r & 15) == 15)
        *reinterpret_cast<f32x4 *>(sRef + ((r + 1) >> 4) * D + ch0) = Gv[j] + pre;
    }
    if (rg == 0) *reinterpret_cast<f32x4 *>(sRef + ch0) = zero4();
    __syncthreads();
    // the remaining bound: every 16-token block's summed log-decay >= -80
    if (rg == 0 && in.flags) {
      bool bad = false;
#pragma unroll
      for (int b = 0; b < NRB; ++b) {
        const f32x4 lo = b + 1 < NRB ? *reinterpret_cast<const f32x4 *>(sRef + (b + 1) * D + ch0)
                                     : tot;
        const f32x4 d = lo - *reinterpret_cast<const f32x4 *>(sRef + b * D + ch0);
        bad |= d[0] < -80.f || d[1] < -80.f || d[2] < -80.f || d[3] < -80.f;
      }
      if (bad) atomicOr(in.flags, KDA_FLAG_DECAY_RANGE);
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = r0 + j;
      if (r < C) {
        const bool live = !TAIL || r < n;
        f32x4 qv = live ? to_f32x4(qr[j]) : zero4();
        f32x4 kv = live ? to_f32x4(kr[j]) : zero4();
        const f32x4 vv = live ? to_f32x4(vr[j]) : zero4();
        if (in.l2norm_qk) {
          qv *= l2_inv_norm<CG>(qv);
          kv *= l2_inv_norm<CG>(kv);
        }
        const float br = live ? (in.beta_logits ? sigmoid(brr[j]) : brr[j]) : 0.f;
        if (cg == 0) sBeta[r] = br;
        const f32x4 G = Gv[j] + pre;
        const f32x4 R = *reinterpret_cast<const f32x4 *>(sRef + (r >> 4) * D + ch0);
        f32x4 qt, kt, ktl, qtl, khl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float eg = __expf(G[e]);
          const float el = __expf(G[e] - R[e]);  // <= 1; >= e^-80 inside a block
          const float eh = __builtin_amdgcn_rcpf(el);
          qt[e] = qv[e] * eg;
          kt[e] = kv[e] * eg;
          ktl[e] = kv[e] * el;
          qtl[e] = qv[e] * el;
          khl[e] = kv[e] * eh;
          ke[e][j] = from_f32<T>(kv[e] * __expf(tot[e] - G[e]));
          bk[e][j] = from_f32<T>(br * kt[e]);
          bv[e][j] = from_f32<T>(br * vv[e]);
        }
        // Qt goes out here: sQt holds the block-referenced rows
        store4_f32<T>(qt_tile + frag_off(r, kperm_pos(ch0), D), qt);
        store4_f32<T>(sKt + r * LDR + ch0, ktl);
        store4_f32<T>(sKh + r * LDR + ch0, khl);
        store4_f32<T>(sQt + r * LDR + ch0, qtl);
      }
    }
  };
  if (n == C)
    scaled_rows(Flag<false>{});
  else
    scaled_rows(Flag<true>{});
  if (__builtin_expect(far, 0)) far_rows(far_pre, far_tot);
  __syncthreads();

  // ---------------- phase 2: Qt out; A and P on the matrix cores ------------
  // Qt leaves from LDS one contiguous 16 x 32 fragment block per wavefront
  // store (rows past the chunk end are zero).
  if (!far) {
    for (int b = wv; b < Cfg::NQB; b += NW) {
      const int rb = b / KD, ks = b % KD;
      copy_run<T>(qt_tile + b * 512 + lane * 8, sQt + (16 * rb + lr) * LDR + 32 * ks + 4 * lg);
    }
  }
  // Each wave takes a token block and a pair of key blocks 2m, 2m + 1, whose
  // P columns are adjacent kperm positions: one 16-byte store per lane.
  // Every tile is computed, also those above the diagonal (masked to zero
  // below; padding key blocks read a clamped in-chunk row): a branch between a
  // matrix-core instruction and the reads of its result has been seen to
  // return a stale register on gfx950, so results are only ever read in
  // straight-line code after the instructions that produce them.
  T *p_tile = p_out + tile * (C * CK);
  // FAR: the row operands are scaled by e^(R_rb - R_kb) per channel for key
  // block kb (1 on and above the diagonal blocks, which are masked anyway).
  auto ap_tiles = [&](auto far_form) {
  constexpr bool FAR = decltype(far_form)::value;
  // (the rare FAR form is kept compact: its loops are not unrolled)
#pragma unroll FAR ? 1 : 2
  for (int it = 0; it < (Cfg::NP + NW - 1) / NW; ++it) {
    const int idx = wv + NW * it;
    if (idx >= Cfg::NP) break;
    const int rb = idx / (NKB / 2), m = idx % (NKB / 2);
    const int hrow0 = min(32 * m + lr, C - 1), hrow1 = min(32 * m + 16 + lr, C - 1);
    f32x4 accA0 = zero4(), accA1 = zero4(), accP0 = zero4(), accP1 = zero4();
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      const int kk = 32 * ks + 8 * lg;
      const F fk = load8<T>(sKt + (16 * rb + lr) * LDR + kk);
      const F fq = load8<T>(sQt + (16 * rb + lr) * LDR + kk);
      const F fh0 = load8<T>(sKh + hrow0 * LDR + kk);
      const F fh1 = load8<T>(sKh + hrow1 * LDR + kk);
      if constexpr (FAR) {
        const float *rr = sRef + rb * D + kk;
        const float *r0p = sRef + min(2 * m, NRB - 1) * D + kk;
        const float *r1p = sRef + min(2 * m + 1, NRB - 1) * D + kk;
        F fk0, fk1, fq0, fq1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s0 = __expf(fminf(rr[e] - r0p[e], 0.f));
          const float s1 = __expf(fminf(rr[e] - r1p[e], 0.f));
          fk0[e] = from_f32<T>(to_f32(fk[e]) * s0);
          fk1[e] = from_f32<T>(to_f32(fk[e]) * s1);
          fq0[e] = from_f32<T>(to_f32(fq[e]) * s0);
          fq1[e] = from_f32<T>(to_f32(fq[e]) * s1);
        }
        accA0 = mma_k32(fk0, fh0, accA0);
        accA1 = mma_k32(fk1, fh1, accA1);
        accP0 = mma_k32(fh0, fq0, accP0);
        accP1 = mma_k32(fh1, fq1, accP1);
      } else {
        accA0 = mma_k32(fk, fh0, accA0);  // A[16 rb + 4 lg + i][32 m + lr]
        accA1 = mma_k32(fk, fh1, accA1);  // A[16 rb + 4 lg + i][32 m + 16 + lr]
        accP0 = mma_k32(fh0, fq, accP0);  // P[16 rb + lr][32 m + 4 lg + i]
        accP1 = mma_k32(fh1, fq, accP1);  // P[16 rb + lr][32 m + 16 + 4 lg + i]
      }
    }
    f32x4 bta;
#pragma unroll
    for (int i = 0; i < 4; ++i) bta[i] = sBeta[16 * rb + 4 * lg + i];
    const f32x4 av0 = accA0 * bta, av1 = accA1 * bta;  // branch-free: masks are selects
    const int prow = 16 * rb + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int arow = 16 * rb + 4 * lg + i;
      sA[arow * LDA + 32 * m + lr] = (32 * m + lr < arow) ? av0[i] : 0.f;
      sA[arow * LDA + 32 * m + 16 + lr] = (32 * m + 16 + lr < arow) ? av1[i] : 0.f;
      accP0[i] = (32 * m + 4 * lg + i <= prow) ? accP0[i] : 0.f;
      accP1[i] = (32 * m + 16 + 4 * lg + i <= prow) ? accP1[i] : 0.f;
    }
    // A pair of key blocks that starts past the token block's last row is
    // zero; the inter-chunk kernel never loads it, so it is not stored
    // (a quarter of P's bytes when C = 64).  The empty asm makes the masked
    // results exist before the branch, so the compiler cannot move the reads
    // of the matrix-core registers behind it.
    asm volatile("" ::"v"(accP0), "v"(accP1));
    if (32 * m <= 16 * rb + 15)
      store8_f32<T>(p_tile + frag_off(prow, 32 * m + 8 * lg, CK), accP0, accP1);
  }
  };
  if constexpr (NRB > 1) {
    if (__builtin_expect(far, 0))
      ap_tiles(Flag<true>{});
    else
      ap_tiles(Flag<false>{});
  } else {  // one block per chunk: the block reference is the chunk start
    ap_tiles(Flag<false>{});
  }
  __syncthreads();

  // ---------------- phase 3: staged B operands, T = (I + A)^-1 ---------------
  if (r0 < C) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      store_run<T, RPT>(sBKt + (ch0 + e) * LDT + r0, bk[e]);
      store_run<T, RPT>(sBVt + (ch0 + e) * LDT + r0, bv[e]);
      store_run<T, RPT>(sKeT + (ch0 + e) * LDT + r0, ke[e]);
    }
  }
  if (CK > C) {  // padding tokens are zero
    for (int e = tid; e < D * (CK - C); e += NT) {
      const int ch = e / (CK - C), r = C + e % (CK - C);
      sBKt[ch * LDT + r] = from_f32<T>(0.f);
      sBVt[ch * LDT + r] = from_f32<T>(0.f);
      sKeT[ch * LDT + r] = from_f32<T>(0.f);
    }
  }
  // diagonal 16 x 16 blocks: lane j of wave b computes column j of T_bb by
  // forward substitution, right-looking: once T[m][j] is known it is added
  // into every later row's sum, so a step waits on one multiply-add (the
  // sums take their terms in the same order as a row-by-row substitution)
  if (wv < NRB && lane < 16) {
    const int b0 = 16 * wv, jcol = lane;
    float acc[16], tcol[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      tcol[m] = jcol < m ? -acc[m] : (m == jcol ? 1.f : 0.f);
#pragma unroll
      for (int r = m + 1; r < 16; ++r) acc[r] += sA[(b0 + r) * LDA + b0 + m] * tcol[m];
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) sA[(b0 + m) * LDA + b0 + jcol] = tcol[m];
  }
  __syncthreads();
  // blocks below the diagonal: T_ij = -T_ii X, X = sum_{m=j}^{i-1} A_im T_mj.
  // Block column j needs only T blocks of column j, so wave j walks its
  // column down alone, with no barrier between block rows.  T_ij overwrites
  // A_ij, which the walks of the columns left of j still read: each wave
  // first copies the A and T_ii fragments of its walk into registers, and
  // one barrier separates those reads from every write.  Each column is its
  // own fully unrolled code, so matrix-core results are read in straight-line
  // code; the products take their terms in block-row order as before.
  static_assert(NRB <= NW, "one wave per block column");
  constexpr int NPAIR = NRB * (NRB - 1) / 2;  // (i, m) pairs of column 0
  f32x4 aF[NPAIR > 0 ? NPAIR : 1], tF[NRB > 1 ? NRB - 1 : 1];
  auto col_load = [&](auto col) {
    constexpr int bj = decltype(col)::value;
    int q = 0;
#pragma unroll
    for (int bi = bj + 1; bi < NRB; ++bi) {
      tF[bi - bj - 1] =
          *reinterpret_cast<const f32x4 *>(sA + (16 * bi + lr) * LDA + 16 * bi + 4 * lg);
#pragma unroll
      for (int m = bj; m < bi; ++m, ++q)
        aF[q] = *reinterpret_cast<const f32x4 *>(sA + (16 * bi + lr) * LDA + 16 * m + 4 * lg);
    }
  };
  auto col_walk = [&](auto col) {
    constexpr int bj = decltype(col)::value;
    int q = 0;
#pragma unroll
    for (int bi = bj + 1; bi < NRB; ++bi) {
      f32x4 X = zero4();
#pragma unroll
      for (int m = bj; m < bi; ++m, ++q) {
        f32x4 bf;
#pragma unroll
        for (int i = 0; i < 4; ++i) bf[i] = sA[(16 * m + 4 * lg + i) * LDA + 16 * bj + lr];
        X = mma_f32_k16(aF[q], bf, X);
      }
      const f32x4 Y = mma_f32_k16(tF[bi - bj - 1], X, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) sA[(16 * bi + 4 * lg + i) * LDA + 16 * bj + lr] = -Y[i];
    }
  };
  if constexpr (NRB > 1) {
    if (wv == 0) col_load(std::integral_constant<int, 0>{});
    if constexpr (NRB > 2) {
      if (wv == 1) col_load(std::integral_constant<int, 1>{});
    }
    if constexpr (NRB > 3) {
      if (wv == 2) col_load(std::integral_constant<int, 2>{});
    }
    __syncthreads();
    if (wv == 0) col_walk(std::integral_constant<int, 0>{});
    if constexpr (NRB > 2) {
      if (wv == 1) col_walk(std::integral_constant<int, 1>{});
    }
    if constexpr (NRB > 3) {
      if (wv == 2) col_walk(std::integral_constant<int, 2>{});
    }
    __syncthreads();
  }

  // ---------------- phase 4: W^T and U on the matrix cores -------------------
  // For token block rb the T fragment (row 16 rb + lr, K-slot 8 lg..) is the
  // A operand of U = T (Diag(beta) V) and the B operand of
  // W^T = (Diag(beta) Kt)^T T^T.
  T *ke_tile = ket_out + tile * (D * CK);
  for (int b = wv; b < Cfg::NEB; b += NW) {  // Ke^T blocks, as Qt in phase 2
    const int cb = b / KC, ks = b % KC;
    copy_run<T>(ke_tile + b * 512 + lane * 8, sKeT + (16 * cb + lr) * LDT + 32 * ks + 4 * lg);
  }
  T *w_tile = w_out + tile * (C * D);
  T *ut_tile = ut_out + tile * (D * C);
  {
    constexpr int CPW = Cfg::CPW;
    const int rb = wv % NRB, cb0 = (wv / NRB) * CPW;
    F tf[KC];
#pragma unroll
    for (int ks = 0; ks < KC; ++ks)
      tf[ks] = frag_from_f32<T>(sA + (16 * rb + lr) * LDA + 32 * ks + 8 * lg);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int cb = cb0 + j;
      if (CPW * Cfg::WPR != NCB && cb >= NCB) break;  // uniform
      f32x4 accW = zero4(), accU = zero4();
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) {  // all K-steps: T is zero above its diagonal
        const int kk = 32 * ks + 8 * lg;
        accW = mma_k32(load8<T>(sBKt + (16 * cb + lr) * LDT + kk), tf[ks], accW);
        accU = mma_k32(tf[ks], load8<T>(sBVt + (16 * cb + lr) * LDT + kk), accU);
      }
      // accW[i] = W[16 rb + lr][16 cb + 4 lg + i]; accU[i] = U[16 rb + 4 lg + i][16 cb + lr]
      store4_f32<T>(w_tile + frag_off(16 * rb + lr, kperm_pos(16 * cb + 4 * lg), D), accW);
      store4_f32<T>(ut_tile + tile_off(16 * rb + 4 * lg, 16 * cb + lr, C), accU);
    }
  }
}

template <typename T, int D, int C, bool RAW>
static hipError_t launch_intra_t(const FwdArgs &a) {
  using Cfg = IntraCfg<T, D, C>;
  auto kern = intra_chunk_kernel<T, D, C, RAW>;
  static std::atomic<unsigned long long> lds_raised{0};
  const hipError_t attr = raise_lds_limit((const void *)kern, Cfg::LDS_BYTES, lds_raised);
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)a.grid_chunks * (unsigned)a.num_heads);
  char *ws = a.ws;
  hipLaunchKernelGGL(kern, grid, dim3(Cfg::NT), Cfg::LDS_BYTES, a.stream,
                     reinterpret_cast<const T *>(a.q), reinterpret_cast<const T *>(a.k),
                     reinterpret_cast<const T *>(a.v), a.gate, a.beta, a.in, a.chunk_tab,
                     a.num_seqs, a.num_heads, a.seq_len,
                     reinterpret_cast<T *>(ws + a.lay.qt), reinterpret_cast<T *>(ws + a.lay.w),
                     reinterpret_cast<T *>(ws + a.lay.ut), reinterpret_cast<T *>(ws + a.lay.ket),
                     reinterpret_cast<T *>(ws + a.lay.p), reinterpret_cast<float *>(ws + a.lay.gam));
  return hipGetLastError();
}

template <typename T, int D, int C>
static hipError_t launch_intra_c(const FwdArgs &a) {
  return a.in.gate == KDA_GATE_LOG_ALPHA ? launch_intra_t<T, D, C, false>(a)
                                         : launch_intra_t<T, D, C, true>(a);
}

template <typename T, int D>
static hipError_t launch_intra_d(const FwdArgs &a) {
  switch (a.chunk) {
    case 16: return launch_intra_c<T, D, 16>(a);
    case 32: return launch_intra_c<T, D, 32>(a);
    case 64: return launch_intra_c<T, D, 64>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_intra(const FwdArgs &a, kda_dtype dt) {
  if (a.grid_chunks == 0) return hipSuccess;
  if (dt == KDA_DTYPE_BF16) {
    switch (a.d) {
      case 32: return launch_intra_d<bf16, 32>(a);
      case 64: return launch_intra_d<bf16, 64>(a);
      case 128: return launch_intra_d<bf16, 128>(a);
    }
  } else {
    switch (a.d) {
      case 32: return launch_intra_d<float, 32>(a);
      case 64: return launch_intra_d<float, 64>(a);
      case 128: return launch_intra_d<float, 128>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
