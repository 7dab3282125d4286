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
// independently: a workgroup owns one (sequence, head, column slice of 16,
// 32 or 64 columns) and walks that sequence's chunks.  Its four wavefronts
// split the rows: wave w computes token block w of Unew and O and channel
// blocks w*CBW.. of S, so all four SIMDs issue matrix-core work and each
// wave loads only its quarter of W, Qt, P and Ke.  The blocks meet through
// two tiny LDS exchanges per chunk (Unew after its product, S after the
// update), each a plain lane-for-lane copy: the intra-chunk kernel stores W,
// Qt (channels) and Ke^T, P (tokens) with their contraction index in the
// kperm order of kda_common.hpp, in which a 16x16 output tile held by one
// wave is already half of another wave's K-step operand.  The fp32 state
// stays in registers.
//
// The intra-chunk kernel stores all of these operands fragment-major
// (frag_off / tile_off), so every load below is one contiguous run per wave.
// Loads are the bottleneck of a serial chain: each wave keeps PF = 3 chunks
// of its operands in flight (a ring of register buffers, the loop unrolled
// by 3), requesting chunk c + 3 right after the last use of chunk c's group.
// Short sequences take PF = 1, one buffer (see the launch).
// The requests are unconditional (chunks past the end re-read the last one)
// and fenced with scheduling barriers so the compiler keeps them in place.
// Workgroups of one (sequence, head) share blockIdx % 8 and therefore one
// XCD and its L2, which serves the same W/Qt/Ke/P rows to all slices.
// For bf16 operands with d = 128 and C = 64 on 16-column ring slices the
// launch takes inter_split_kernel instead: the same chain with eight
// wavefronts, four for Unew and O and four that own S (see there).
// The output tile leaves in one of three forms (WIDE_O, DEFER_O below):
// 16-byte row pieces of each wave's rows through LDS on wider slices and in
// the one-buffer form; 16-byte row pieces of the whole tile, deferred to
// the top of the next step, on the other 16-column ring slices without
// warm-up loads; two-byte stores straight from the output tiles on the
// long chains that take warm-up loads.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <bool B>
struct StepKind {
  static constexpr bool value = B;
};

template <typename T, int D, int C, int CT>
struct InterOps {
  using F = typename Frag<T>::type;
  using V4 = typename Vec4<T>::type;
  static constexpr int NCB = D / 16;
  static constexpr int CK = C < 32 ? 32 : C;
  static constexpr int KD = D / 32;
  static constexpr int KC = CK / 32;
  static constexpr int CBW = (NCB + 3) / 4;  // state channel blocks per wave
  // one chunk's operands for one wave
  struct Buf {
    F wA[KD];       // W rows of the wave's token block (K = channels)
    F qA[KD];       // Qt rows of the wave's token block
    F pA[KC];       // P rows of the wave's token block (K = tokens)
    V4 uv[CT];      // U of the wave's token block, one output tile per column tile
    F kA[CBW][KC];  // Ke^T rows of the wave's channel blocks (K = tokens)
    float gl;       // e^{G_n}: lane 16 j + r holds channel 16 cb_j + r (cb_j = wave's jth block)
    int warm;       // L2 warm-up load of a later chunk (WARM only)
  };
};

// CT: 16-column tiles per workgroup (a slice of 16 CT columns).  The tiles
// share every W, Qt, P and Ke^T fragment a wave loads, so wider slices halve
// the operand bytes per column but lengthen each serial step; the launch
// takes them only where they cut the rounds of workgroups on the GPU.
//
// WARM: L2 warm-up loads.  Every slice of a (sequence, head) reads the same
// W, Qt, Ke^T and P lines, and the first to ask for a line waits for HBM.
// With WARM each workgroup also reads one dword from each of its 1/NS share
// of those lines, WARM_AHEAD chunks beyond its register ring, so that the
// ring's own loads find the lines in the XCD's L2.  The value read only
// feeds an empty asm statement at the end.  It pays on long chains of
// 16-column slices (measured on MI355X: the B=1 H=32 T=32768 prefill's chain
// 549 -> 522 us) and costs time on short chains and wide slices, so the
// launch enables it only there.
constexpr int WARM_AHEAD = 3;

template <typename T, int D, int C, int PF, int CT, bool WARM>
__global__ __launch_bounds__(256) void inter_chunk_kernel(
    const T *__restrict__ qt, const T *__restrict__ w, const T *__restrict__ ut,
    const T *__restrict__ ket, const T *__restrict__ pm,
    const float *__restrict__ gam, const int *__restrict__ cu,
    const int *__restrict__ seq_first, int N, int H, int seq_len,
    const float *__restrict__ s0, float *__restrict__ s_final,
    const int *__restrict__ slots, int num_slots, const OptArgs in, T *__restrict__ o) {
  using Ops = InterOps<T, D, C, CT>;
  using F = typename Ops::F;
  using V4 = typename Ops::V4;
  using Buf = typename Ops::Buf;
  constexpr int NRB = C / 16, NCB = Ops::NCB, CK = Ops::CK, KD = Ops::KD, KC = Ops::KC;
  constexpr int CBW = Ops::CBW, NS = D / (16 * CT);

  // S (operand type), one output tile per channel block.  The one-buffer
  // form (RE_S) keeps two copies, the chunk's entering S and the updated one,
  // and its output product reads S again from LDS instead of holding it in
  // registers through the step: 20 registers fewer at 16-column slices,
  // which lets four workgroups share a CU instead of three (1,100 short
  // sequences: 967 -> 873 us).  The ring keeps S in registers, measured
  // faster there (less LDS traffic on its longer steps).
  constexpr bool RE_S = PF == 1;
  __shared__ V4 sS[RE_S ? 2 : 1][CT][NCB][64];
  __shared__ V4 sU[CT][2 * KC][64];  // Unew (operand type), one tile per token block
  // Wide output stores (WIDE_O): each wave turns its 16 output rows into
  // 16-byte row pieces through LDS.  The direct form stores 4 CT narrow
  // pieces per lane and step, and every store counts against the wave's
  // 63 outstanding vector-memory operations, which the operand ring needs:
  // at 64-column slices a step would hold 35 of them.  16-column slices of
  // the ring (4 stores per step) keep the direct form, measured no slower.
  constexpr bool WIDE_O = CT >= 2 || PF == 1;
  // Deferred output stores (DEFER_O), for 16-column slices of the ring
  // without warm-up loads (short and mid-length chains): the waves leave
  // their rows in LDS, and after the step's last barrier the whole tile goes
  // out as 16-byte row pieces at the top of the next step, off the output
  // product's path.  B=2 H=8 T=2048: chain 25.8 -> 25.4 us; B=1 H=32 T=4096:
  // 49.8 -> 48.8 us.  With warm-up loads (long chains) it was 9% slower.
  constexpr bool DEFER_O = CT == 1 && PF == 3 && !WARM;
  constexpr int OW = 16 * CT, PE = 16 / (int)sizeof(T), LDO = OW + PE;
  constexpr int PPR = OW / PE, WP = 16 * PPR, WPL = (WP + 63) / 64;
  constexpr int NPC = C * PPR, PPT = (NPC + 255) / 256;  // pieces of the tile, per thread
  __shared__ __align__(16) T sO[(WIDE_O || DEFER_O) ? C : 1][LDO];

  if (inputs_rejected(in)) return;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int slice = local % NS, unit = local / NS;
  const int pair = unit * 8 + xcd;
  if (pair >= N * H) return;
  const int seq = pair / H, h = pair % H;
  const int tid = threadIdx.x, lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());  // scalar: branches stay uniform
  const int lr = lane & 15, lg = lane >> 4;
  const int col0 = slice * 16 * CT;
  // Roles.  With C = 64 and d % 64 == 0 every wave owns a token block and
  // CBW channel blocks and nothing below branches.  Smaller shapes leave some
  // waves without a block; those still load (clamped, in-bounds) operands so
  // that every load stays unconditional, and skip only the arithmetic.
  constexpr bool ALL_RB = NRB >= 4;
  constexpr bool ALL_CB = NCB % 4 == 0;
  const bool has_rb = ALL_RB || wv < NRB;
  const int rb = ALL_RB ? wv : min(wv, NRB - 1);

  int t0, len, first;
  if (cu) {
    t0 = cu[seq];
    len = cu[seq + 1] - t0;
    first = len > 0 ? seq_first[seq] : 0;
  } else {
    t0 = seq * seq_len;
    len = seq_len;
    first = seq * ((seq_len + C - 1) / C);
  }
  const int nch = (len + C - 1) / C;
  const int64_t rs = (int64_t)H * D;
  // state of this (sequence, head): row `pair`, or its slot of the pools
  int64_t spair = pair;
  bool has_state = true;
  if (slots) {
    const int sl = slots[seq];
    has_state = sl >= 0 && sl < num_slots;  // padding: zero start, no final write
    spair = has_state ? (int64_t)sl * H + h : 0;
  }

  // the wave's state: S[j][t][i] = S[16 cb + 4 lg + i][col0 + 16 t + lr], cb = wv CBW + j
  f32x4 S[CBW][CT];
  const int64_t sbase = spair * D * D + col0 + lr;
#pragma unroll
  for (int j = 0; j < CBW; ++j) {
    const int cb = wv * CBW + j;
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      f32x4 x = zero4();
      if (cb < NCB) {
        if (s0 && has_state) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            x[i] = s0[sbase + 16 * t + (int64_t)(16 * cb + 4 * lg + i) * D];
        }
        sS[0][t][cb][lane] = vec4_from_f32<T>(x);
      }
      S[j][t] = x;
    }
  }
  for (int e = tid; e < CT * (2 * KC - NRB) * 64; e += 256) {  // padding token blocks stay zero
    const int t = e / ((2 * KC - NRB) * 64), r = e % ((2 * KC - NRB) * 64);
    sU[t][NRB + r / 64][r % 64] = vec4_from_f32<T>(zero4());
  }
  __syncthreads();

  auto tile_of = [&](int ci) { return (int64_t)(first + ci) * H + h; };
  auto load_wu = [&](Buf &B, int ci) {
    const int64_t tile = tile_of(ci);
    const T *wt = w + tile * (C * D) + (rb * KD * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) B.wA[ks] = load8<T>(wt + ks * 512);
#pragma unroll
    for (int t = 0; t < CT; ++t)
      B.uv[t] = load4<T>(ut + tile * (D * C) + (((slice * CT + t) * NRB + rb) * 64 + lane) * 4);
  };
  auto load_qp = [&](Buf &B, int ci) {
    const int64_t tile = tile_of(ci);
    const T *qq = qt + tile * (C * D) + (rb * KD * 64 + lane) * 8;
    const T *pp = pm + tile * (C * CK) + (rb * KC * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) B.qA[ks] = load8<T>(qq + ks * 512);
    // P is lower triangular: a token K-step that starts past the wave's last
    // row is zero and is not loaded (saves a quarter of P's bytes when C = 64)
#pragma unroll
    for (int ks = 0; ks < KC; ++ks) {
      if (32 * ks <= 16 * rb + 15) B.pA[ks] = load8<T>(pp + ks * 512);
      else B.pA[ks] = F{};
    }
  };
  auto load_kg = [&](Buf &B, int ci) {
    const int64_t tile = tile_of(ci);
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = ALL_CB ? wv * CBW + j : min(wv * CBW + j, NCB - 1);
      const T *kk = ket + tile * (D * CK) + (cb * KC * 64 + lane) * 8;
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) B.kA[j][ks] = load8<T>(kk + ks * 512);
    }
    // e^{G_n} of the wave's CBW channel blocks, one dword per lane (lanes past
    // them repeat the last block); the step gathers each lane's 4 rows with
    // lane permutes.  A 16-byte load per lane, 16 lanes to an address, would
    // return 16x the bytes through the vector-memory path.
    {
      const int jl = min(lane >> 4, CBW - 1);
      const int cbl = ALL_CB ? wv * CBW + jl : min(wv * CBW + jl, NCB - 1);
      B.gl = gam[tile * D + 16 * cbl + (lane & 15)];
    }
  };
  auto load_all = [&](Buf &B, int ci) {
    load_wu(B, ci);
    load_qp(B, ci);
    load_kg(B, ci);
  };
  // warm-up line of this lane: line li of the tile's W, Qt, Ke^T and P lines
  // taken in that order (lanes past the workgroup's share repeat its last
  // line; the loads of one instruction to one line merge)
  constexpr int LQ = C * D * (int)sizeof(T) / 128, LK = D * CK * (int)sizeof(T) / 128,
                LP = C * CK * (int)sizeof(T) / 128, NL = 2 * LQ + LK + LP;
  constexpr int NLW = (NL + NS - 1) / NS, NLV = (NLW + 3) / 4;
  static_assert(!WARM || NLV <= 64, "one warm-up load per wave and chunk");
  const int wli = min(slice * NLW + wv * NLV + min(lane, NLV - 1), NL - 1);
  auto warm_load = [&](int ci) -> int {
    const int64_t tile = tile_of(ci);
    const char *p;
    if (wli < LQ)
      p = reinterpret_cast<const char *>(w + tile * (C * D)) + wli * 128;
    else if (wli < 2 * LQ)
      p = reinterpret_cast<const char *>(qt + tile * (C * D)) + (wli - LQ) * 128;
    else if (wli < 2 * LQ + LK)
      p = reinterpret_cast<const char *>(ket + tile * (D * CK)) + (wli - 2 * LQ) * 128;
    else
      p = reinterpret_cast<const char *>(pm + tile * (C * CK)) + (wli - 2 * LQ - LK) * 128;
    return *reinterpret_cast<const int *>(p);
  };
  int warm_sink = 0;

  // FULL: a chunk of C rows (every chunk but a sequence's last), whose o
  // stores need no row mask.
  // DEFER_O: the previous step's output tile, from LDS to o
  int prev_tc = 0, prev_rows = 0;
  auto flush_o = [&]() {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int e = tid + 256 * p;
      if (NPC % 256 == 0 || e < NPC) {
        const int r = e / PPR, c = (e % PPR) * PE;
        if (r < prev_rows)
          *reinterpret_cast<uint4 *>(o + (int64_t)(prev_tc + r) * rs + (int64_t)h * D + col0 + c) =
              *reinterpret_cast<const uint4 *>(&sO[r][c]);
      }
    }
  };
  auto step = [&](Buf &B, int ci, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const int nxt = min(ci + PF, nch - 1);
    const int tc = t0 + ci * C;
    const int rows = FULL ? C : min(C, len - ci * C);
    if constexpr (DEFER_O) {  // the last step's barrier made its rows visible
      flush_o();
      prev_tc = tc;
      prev_rows = rows;
    }

    // S entering the chunk, as K-step operands over channels, per column tile
    const int cur = RE_S ? (ci & 1) : 0;
    auto s_operand = [&](int t, int ks) {
      return join4(sS[cur][t][2 * ks][lane], sS[cur][t][2 * ks + 1][lane]);
    };
    F sb[CT][KD];
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) sb[t][ks] = s_operand(t, ks);

    // Unew = U - W S for the wave's token block (two accumulators per tile)
    if (has_rb) {
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
          if (ks & 1) a1 = mma_k32(B.wA[ks], sb[t][ks], a1);
          else a0 = mma_k32(B.wA[ks], sb[t][ks], a0);
        }
        sU[t][rb][lane] = vec4_from_f32<T>(to_f32x4(B.uv[t]) - (a0 + a1));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_wu(B, nxt);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();

    // Unew of the whole chunk as K-step operands over tokens, per column tile
    F ub[CT][KC];
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int ks = 0; ks < KC; ++ks)
        ub[t][ks] = join4(sU[t][2 * ks][lane], sU[t][2 * ks + 1][lane]);

    // S <- Diag(e^{G_n}) S + Ke^T Unew for the wave's channel blocks
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (ALL_CB || cb < NCB) {
        f32x4 gj;  // e^{G_n} of rows 16 cb + 4 lg + i
#pragma unroll
        for (int i = 0; i < 4; ++i)
          gj[i] = __int_as_float(
              __builtin_amdgcn_ds_bpermute((16 * j + 4 * lg + i) * 4, __float_as_int(B.gl)));
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          f32x4 acc = S[j][t] * gj;
#pragma unroll
          for (int ks = 0; ks < KC; ++ks) acc = mma_k32(B.kA[j][ks], ub[t][ks], acc);
          S[j][t] = acc;
          sS[RE_S ? cur ^ 1 : 0][t][cb][lane] = vec4_from_f32<T>(acc);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_kg(B, nxt);
    __builtin_amdgcn_sched_barrier(0);

    // O = Qt S + P Unew for the wave's token block
    if (has_rb) {
      V4 ov[CT];
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        f32x4 oc = zero4();
#pragma unroll
        for (int ks = 0; ks < KD; ++ks)
          oc = mma_k32(B.qA[ks], RE_S ? s_operand(t, ks) : sb[t][ks], oc);
#pragma unroll
        for (int ks = 0; ks < KC; ++ks) oc = mma_k32(B.pA[ks], ub[t][ks], oc);
        // read (and convert) before any branch: matrix-core results are read
        // only in straight-line code after the instructions that produce them;
        // "+ 0" makes it a real VALU read also when T is fp32
        ov[t] = vec4_from_f32<T>(oc + 0.f);
      }
      if constexpr (WIDE_O) {
        // the wave's rows only, so no other wave takes part: LDS operations
        // of one wave complete in order
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) sO[16 * rb + 4 * lg + i][16 * t + lr] = ov[t][i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < WPL; ++p) {
          const int e = lane + 64 * p;
          if (WP % 64 == 0 || e < WP) {
            const int row = 16 * rb + e / PPR, c = (e % PPR) * PE;
            if (FULL || row < rows)
              *reinterpret_cast<uint4 *>(o + (int64_t)(tc + row) * rs + (int64_t)h * D + col0 +
                                         c) = *reinterpret_cast<const uint4 *>(&sO[row][c]);
          }
        }
      } else if constexpr (DEFER_O) {
        // rewritten only after this step's first barrier, which every
        // wave passes after its flush of the previous tile
#pragma unroll
        for (int i = 0; i < 4; ++i) sO[16 * rb + 4 * lg + i][lr] = ov[0][i];
      } else {
        T *op = o + (int64_t)(tc + 16 * rb + 4 * lg) * rs + (int64_t)h * D + col0 + lr;
        if (FULL || rows == C) {
#pragma unroll
          for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) op[i * rs + 16 * t] = ov[t][i];
        } else {
#pragma unroll
          for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * rb + 4 * lg + i < rows) op[i * rs + 16 * t] = ov[t][i];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_qp(B, nxt);
    if constexpr (WARM) {  // the warm-up load issued PF steps ago has landed
      warm_sink ^= B.warm;
      B.warm = warm_load(min(ci + PF + WARM_AHEAD, nch - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  };

  static_assert(PF == 1 || PF == 3, "one operand buffer, or a ring of three");
  static_assert(!WARM || PF == 3, "warm-up loads ride on the ring");
  if constexpr (PF == 1) {
    // One buffer: each group of the next chunk's operands is requested right
    // after its last use in this chunk.  About 130 registers fewer per lane
    // than the ring, so more workgroups share a CU: for sequences of a few
    // chunks, where no ring fills, that overlap is what counts.
    Buf B0;
    B0.warm = 0;
    if (nch > 0) load_all(B0, 0);
    const int nfull = len / C;
    int ci = 0;
    for (; ci < nfull; ++ci) step(B0, ci, StepKind<true>{});
    if (ci < nch) step(B0, ci, StepKind<false>{});
  } else {
    Buf B0, B1, B2;
    B0.warm = B1.warm = B2.warm = 0;
    if (nch > 0) {
      load_all(B0, 0);
      load_all(B1, min(1, nch - 1));
      load_all(B2, min(2, nch - 1));
      if constexpr (WARM) {
        B0.warm = warm_load(min(PF, nch - 1));
        B1.warm = warm_load(min(PF + 1, nch - 1));
        B2.warm = warm_load(min(PF + 2, nch - 1));
      }
    }
    // Full chunks three at a time with nothing conditional in the loop body:
    // every pass issues the same loads and stores, so the waits the compiler
    // places for a buffer's loads leave the other two chunks' loads in flight
    // (conditional steps inside the loop made one step in three wait for the
    // next chunk's loads as well).  The last one to three chunks, the partial
    // one included, follow the loop.
    const int nfull = len / C;
    int ci = 0;
    for (; ci + 3 <= nfull; ci += 3) {
      step(B0, ci, StepKind<true>{});
      step(B1, ci + 1, StepKind<true>{});
      step(B2, ci + 2, StepKind<true>{});
    }
    if (ci < nch) step(B0, ci, StepKind<false>{});
    if (ci + 1 < nch) step(B1, ci + 1, StepKind<false>{});
    if (ci + 2 < nch) step(B2, ci + 2, StepKind<false>{});

    if constexpr (WARM) {
      warm_sink ^= B0.warm ^ B1.warm ^ B2.warm;
      asm volatile("" ::"v"(warm_sink));
    }
  }

  if constexpr (DEFER_O) flush_o();  // the last chunk's tile
  if (s_final && has_state) {
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = wv * CBW + j;
      if (cb < NCB) {
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s_final[sbase + 16 * t + (int64_t)(16 * cb + 4 * lg + i) * D] = S[j][t][i];
      }
    }
  }
}

// Split-role form of the same chain, for 16-column slices of bf16 operands
// with d = 128 and C = 64.  Eight wavefronts: waves 0-3 (the output role)
// each own a token block rb and compute Unew = U - W S and O = Qt S + P Unew
// for it; waves 4-7 (the state role) each own two channel blocks of S and
// compute S <- Diag(e^{G_n}) S + Ke^T Unew.  The output product and the
// state update then run side by side after the step's first barrier
// instead of one after the other in the same waves, and eight waves issue
// the step's loads.  The LDS exchanges, their barriers (two per step,
// executed by every wave) and the fragment loads are those of
// inter_chunk_kernel.
template <typename T, int D, int C, bool WARM>
__global__ __launch_bounds__(512) void inter_split_kernel(
    const T *__restrict__ qt, const T *__restrict__ w, const T *__restrict__ ut,
    const T *__restrict__ ket, const T *__restrict__ pm,
    const float *__restrict__ gam, const int *__restrict__ cu,
    const int *__restrict__ seq_first, int N, int H, int seq_len,
    const float *__restrict__ s0, float *__restrict__ s_final,
    const int *__restrict__ slots, int num_slots, const OptArgs in, T *__restrict__ o) {
  using F = typename Frag<T>::type;
  using V4 = typename Vec4<T>::type;
  constexpr int NRB = C / 16, NCB = D / 16, CK = C, KD = D / 32, KC = C / 32;
  constexpr int CBW = NCB / 4, NS = D / 16;
  static_assert(NRB == 4 && NCB % 4 == 0 && C == 64, "four token blocks, whole channel blocks");
  __shared__ V4 sS[NCB][64];  // S (operand type), one tile per channel block
  __shared__ V4 sU[NRB][64];  // Unew (operand type), one tile per token block
  // Long chains (WARM) store each wave's output tile as 16-byte row pieces
  // through LDS: a quarter of the store instructions through the vector-
  // memory path that bounds the step (long chain 481.8 -> 478.2 us); on
  // shorter chains the direct two-byte stores measured faster (23.3 vs 24.3 us).
  constexpr bool WO = WARM;
  constexpr int LDO = 16 + 16 / (int)sizeof(T);  // padded row of a wave's output tile
  __shared__ __align__(16) T sO[WO ? 4 : 1][16][WO ? LDO : 1];

  if (inputs_rejected(in)) return;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int slice = local % NS, unit = local / NS;
  const int pair = unit * 8 + xcd;
  if (pair >= N * H) return;
  const int seq = pair / H, h = pair % H;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());  // 0 .. 7
  const bool out_role = wv < 4;
  const int rw = out_role ? wv : wv - 4;  // token block (output) or channel-block group (state)
  const int lr = lane & 15, lg = lane >> 4;
  const int col0 = slice * 16;

  int t0, len, first;
  if (cu) {
    t0 = cu[seq];
    len = cu[seq + 1] - t0;
    first = len > 0 ? seq_first[seq] : 0;
  } else {
    t0 = seq * seq_len;
    len = seq_len;
    first = seq * ((seq_len + C - 1) / C);
  }
  const int nch = (len + C - 1) / C;
  const int64_t rs = (int64_t)H * D;
  int64_t spair = pair;
  bool has_state = true;
  if (slots) {
    const int sl = slots[seq];
    has_state = sl >= 0 && sl < num_slots;  // padding: zero start, no final write
    spair = has_state ? (int64_t)sl * H + h : 0;
  }

  // the state role's channel blocks: S[j][i] = S[16 cb + 4 lg + i][col0 + lr], cb = rw CBW + j
  f32x4 S[CBW];
  const int64_t sbase = spair * D * D + col0 + lr;
#pragma unroll
  for (int j = 0; j < CBW; ++j) {
    S[j] = zero4();
    if (!out_role) {
      const int cb = rw * CBW + j;
      if (s0 && has_state) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[j][i] = s0[sbase + (int64_t)(16 * cb + 4 * lg + i) * D];
      }
      sS[cb][lane] = vec4_from_f32<T>(S[j]);
    }
  }
  __syncthreads();

  // One chunk's operands for one wave: the output role's W, U, Qt and P rows
  // of its token block, or the state role's Ke^T rows and e^{G_n}.  Each
  // role runs its own copy of the chunk loop below (same steps, same two
  // barriers per step), so that its register ring holds only its operands.
  struct BufO {
    F wA[KD], qA[KD], pA[KC];
    V4 uv;
  };
  struct BufS {
    F kA[CBW][KC];
    float gl;
    int warm;
  };
  auto tile_of = [&](int ci) { return (int64_t)(first + ci) * H + h; };
  auto load_wu = [&](BufO &B, int ci) {
    const int64_t tile = tile_of(ci);
    const T *wt = w + tile * (C * D) + (rw * KD * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) B.wA[ks] = load8<T>(wt + ks * 512);
    B.uv = load4<T>(ut + tile * (D * C) + ((slice * NRB + rw) * 64 + lane) * 4);
  };
  auto load_qp = [&](BufO &B, int ci) {
    const int64_t tile = tile_of(ci);
    const T *qq = qt + tile * (C * D) + (rw * KD * 64 + lane) * 8;
    const T *pp = pm + tile * (C * CK) + (rw * KC * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) B.qA[ks] = load8<T>(qq + ks * 512);
#pragma unroll
    for (int ks = 0; ks < KC; ++ks) {  // P's zero K-steps past the block's last row are not loaded
      if (32 * ks <= 16 * rw + 15) B.pA[ks] = load8<T>(pp + ks * 512);
      else B.pA[ks] = F{};
    }
  };
  auto load_kg = [&](BufS &B, int ci) {
    const int64_t tile = tile_of(ci);
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const T *kk = ket + tile * (D * CK) + ((rw * CBW + j) * KC * 64 + lane) * 8;
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) B.kA[j][ks] = load8<T>(kk + ks * 512);
    }
    B.gl = gam[tile * D + 16 * (rw * CBW + min(lane >> 4, CBW - 1)) + (lane & 15)];
  };
  // L2 warm-up (WARM): the state role reads one dword of each line of its
  // slice's share of a later chunk's W, Qt, Ke^T and P lines
  constexpr int LQ = C * D * (int)sizeof(T) / 128, LK = D * CK * (int)sizeof(T) / 128,
                LP = C * CK * (int)sizeof(T) / 128, NL = 2 * LQ + LK + LP;
  constexpr int NLW = (NL + NS - 1) / NS, NLV = (NLW + 3) / 4;
  static_assert(!WARM || NLV <= 64, "one warm-up load per wave and chunk");
  const int wli = min(slice * NLW + rw * NLV + min(lane, NLV - 1), NL - 1);
  // and the slice's own U lines (2 KiB per chunk: 16 lines, 4 per state
  // wave) in lanes NLV ..; no other slice reads them, so without this their
  // every load waits for HBM (long chain 496 -> 481 us)
  constexpr int LUW = C * 16 * (int)sizeof(T) / 128 / 4;
  static_assert(NLV + LUW <= 64, "warm-up lanes");
  const bool wu_lane = lane >= NLV && lane < NLV + LUW;
  const int wul = rw * LUW + (lane - NLV);
  auto warm_load = [&](int ci) -> int {
    const int64_t tile = tile_of(ci);
    const char *p;
    if (wu_lane)
      p = reinterpret_cast<const char *>(ut + tile * (D * C) + slice * NRB * 64 * 4) + wul * 128;
    else if (wli < LQ)
      p = reinterpret_cast<const char *>(w + tile * (C * D)) + wli * 128;
    else if (wli < 2 * LQ)
      p = reinterpret_cast<const char *>(qt + tile * (C * D)) + (wli - LQ) * 128;
    else if (wli < 2 * LQ + LK)
      p = reinterpret_cast<const char *>(ket + tile * (D * CK)) + (wli - 2 * LQ) * 128;
    else
      p = reinterpret_cast<const char *>(pm + tile * (C * CK)) + (wli - 2 * LQ - LK) * 128;
    return *reinterpret_cast<const int *>(p);
  };

  // Full chunks three at a time with nothing conditional in the loop body,
  // then the last one to three chunks (the partial one included).
  const int nfull = len / C;
  auto chunk_loop = [&](auto &B0, auto &B1, auto &B2, auto step) {
    int ci = 0;
    for (; ci + 3 <= nfull; ci += 3) {
      step(B0, ci, StepKind<true>{});
      step(B1, ci + 1, StepKind<true>{});
      step(B2, ci + 2, StepKind<true>{});
    }
    if (ci < nch) step(B0, ci, StepKind<false>{});
    if (ci + 1 < nch) step(B1, ci + 1, StepKind<false>{});
    if (ci + 2 < nch) step(B2, ci + 2, StepKind<false>{});
  };

  if (out_role) {
    auto step = [&](BufO &B, int ci, auto full) {
      constexpr bool FULL = decltype(full)::value;
      const int nxt = min(ci + 3, nch - 1);
      const int tc = t0 + ci * C;
      const int rows = FULL ? C : min(C, len - ci * C);
      // Unew = U - W S for the token block (two accumulators)
      F sb[KD];
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) sb[ks] = join4(sS[2 * ks][lane], sS[2 * ks + 1][lane]);
      f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        if (ks & 1) a1 = mma_k32(B.wA[ks], sb[ks], a1);
        else a0 = mma_k32(B.wA[ks], sb[ks], a0);
      }
      sU[rw][lane] = vec4_from_f32<T>(to_f32x4(B.uv) - (a0 + a1));
      __builtin_amdgcn_sched_barrier(0);
      load_wu(B, nxt);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      // O = Qt S + P Unew for the token block, stored straight from the tile
      F ub[KC];
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) ub[ks] = join4(sU[2 * ks][lane], sU[2 * ks + 1][lane]);
      f32x4 oc = zero4();
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) oc = mma_k32(B.qA[ks], sb[ks], oc);
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) oc = mma_k32(B.pA[ks], ub[ks], oc);
      const V4 ov = vec4_from_f32<T>(oc + 0.f);  // a real VALU read before any branch
      if constexpr (WO) {
        // the wave's 16 x 16 tile through its own LDS rows, out as 16-byte pieces
#pragma unroll
        for (int i = 0; i < 4; ++i) sO[rw][4 * lg + i][lr] = ov[i];
        __builtin_amdgcn_wave_barrier();
        if (lane < 32) {
          const int r = lane >> 1, c8 = 8 * (lane & 1);
          if (FULL || 16 * rw + r < rows)
            *reinterpret_cast<uint4 *>(o + (int64_t)(tc + 16 * rw + r) * rs + (int64_t)h * D + col0 +
                                       c8) = *reinterpret_cast<const uint4 *>(&sO[rw][r][c8]);
        }
      } else {
        T *op = o + (int64_t)(tc + 16 * rw + 4 * lg) * rs + (int64_t)h * D + col0 + lr;
        if (FULL || rows == C) {
#pragma unroll
          for (int i = 0; i < 4; ++i) op[i * rs] = ov[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * rw + 4 * lg + i < rows) op[i * rs] = ov[i];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_qp(B, nxt);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
    };
    BufO B0, B1, B2;
    if (nch > 0) {
      load_wu(B0, 0);
      load_qp(B0, 0);
      load_wu(B1, min(1, nch - 1));
      load_qp(B1, min(1, nch - 1));
      load_wu(B2, min(2, nch - 1));
      load_qp(B2, min(2, nch - 1));
    }
    chunk_loop(B0, B1, B2, step);
  } else {
    int warm_sink = 0;
    auto step = [&](BufS &B, int ci, auto full) {
      const int nxt = min(ci + 3, nch - 1);
      lds_barrier();  // Unew of the chunk is in LDS
      F ub[KC];
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) ub[ks] = join4(sU[2 * ks][lane], sU[2 * ks + 1][lane]);
      // S <- Diag(e^{G_n}) S + Ke^T Unew for the wave's channel blocks
#pragma unroll
      for (int j = 0; j < CBW; ++j) {
        const int cb = rw * CBW + j;
        f32x4 gj;  // e^{G_n} of rows 16 cb + 4 lg + i
#pragma unroll
        for (int i = 0; i < 4; ++i)
          gj[i] = __int_as_float(
              __builtin_amdgcn_ds_bpermute((16 * j + 4 * lg + i) * 4, __float_as_int(B.gl)));
        f32x4 acc = S[j] * gj;
#pragma unroll
        for (int ks = 0; ks < KC; ++ks) acc = mma_k32(B.kA[j][ks], ub[ks], acc);
        S[j] = acc + 0.f;  // a real VALU read before any branch
        sS[cb][lane] = vec4_from_f32<T>(S[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      load_kg(B, nxt);
      if constexpr (WARM) {  // the warm-up load issued three steps ago has landed
        warm_sink ^= B.warm;
        B.warm = warm_load(min(ci + 3 + WARM_AHEAD, nch - 1));
      }
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      (void)full;
    };
    BufS B0, B1, B2;
    B0.warm = B1.warm = B2.warm = 0;
    if (nch > 0) {
      load_kg(B0, 0);
      load_kg(B1, min(1, nch - 1));
      load_kg(B2, min(2, nch - 1));
      if constexpr (WARM) {
        B0.warm = warm_load(min(3, nch - 1));
        B1.warm = warm_load(min(4, nch - 1));
        B2.warm = warm_load(min(5, nch - 1));
      }
    }
    chunk_loop(B0, B1, B2, step);
    if constexpr (WARM) {
      warm_sink ^= B0.warm ^ B1.warm ^ B2.warm;
      asm volatile("" ::"v"(warm_sink));
    }
  }

  if (!out_role && s_final && has_state) {
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
      const int cb = rw * CBW + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) s_final[sbase + (int64_t)(16 * cb + 4 * lg + i) * D] = S[j][i];
    }
  }
}

// Compute units of the current device (0 if unknown), looked up once per
// device ordinal.
int device_cus() {
  static std::atomic<int> cus[64];  // zero-initialised: not looked up yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0 &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <typename T, int D, int C, int CT, int PF, bool WARM>
static hipError_t launch_inter_ct(const FwdArgs &a) {
  constexpr int NS = D / (16 * CT);
  const int pairs = a.num_seqs * a.num_heads;
  const int units = (pairs + 7) / 8;
  const dim3 grid((unsigned)(8 * units * NS));
  char *ws = a.ws;
  hipLaunchKernelGGL((inter_chunk_kernel<T, D, C, PF, CT, WARM>), grid, dim3(256), 0, a.stream,
                     reinterpret_cast<const T *>(ws + a.lay.qt),
                     reinterpret_cast<const T *>(ws + a.lay.w),
                     reinterpret_cast<const T *>(ws + a.lay.ut),
                     reinterpret_cast<const T *>(ws + a.lay.ket),
                     reinterpret_cast<const T *>(ws + a.lay.p),
                     reinterpret_cast<const float *>(ws + a.lay.gam), a.cu_seqlens,
                     reinterpret_cast<const int *>(ws + a.lay.seq_first), a.num_seqs,
                     a.num_heads, a.seq_len, a.s0, a.s_final, a.in.slots, a.in.num_slots,
                     a.in, reinterpret_cast<T *>(a.o));
  return hipGetLastError();
}

template <typename T, int D, int C, bool WARM>
static hipError_t launch_inter_split(const FwdArgs &a) {
  constexpr int NS = D / 16;
  const int pairs = a.num_seqs * a.num_heads;
  const int units = (pairs + 7) / 8;
  const dim3 grid((unsigned)(8 * units * NS));
  char *ws = a.ws;
  hipLaunchKernelGGL((inter_split_kernel<T, D, C, WARM>), grid, dim3(512), 0, a.stream,
                     reinterpret_cast<const T *>(ws + a.lay.qt),
                     reinterpret_cast<const T *>(ws + a.lay.w),
                     reinterpret_cast<const T *>(ws + a.lay.ut),
                     reinterpret_cast<const T *>(ws + a.lay.ket),
                     reinterpret_cast<const T *>(ws + a.lay.p),
                     reinterpret_cast<const float *>(ws + a.lay.gam), a.cu_seqlens,
                     reinterpret_cast<const int *>(ws + a.lay.seq_first), a.num_seqs,
                     a.num_heads, a.seq_len, a.s0, a.s_final, a.in.slots, a.in.num_slots,
                     a.in, reinterpret_cast<T *>(a.o));
  return hipGetLastError();
}

// Slice width: the fewest rounds of workgroups (one per CU at a time), and
// the narrowest slice among equals (shortest dependent chain per chunk).
// fp32 operands at d = 128 keep 16-column slices: the wider slices' fp32
// fragments do not fit the registers.
//
// Sequences of at most two chunks on average (many short prompts) take the
// one-buffer form: no operand ring fills on them, and its lower register
// count (bf16, d = 128: 128 at 16-column and 166 at 32-column slices) runs
// four or three workgroups per CU where the ring allows one.  Their slices
// stay at most 32 columns wide, since 64-column slices keep one workgroup
// per CU in either form.  Measured on 1,100 packed sequences of 1-100
// tokens, 16 heads: 1,310 us with the ring, 873 us in this form; on longer
// chains the ring wins.
template <typename T, int D, int C>
static hipError_t launch_inter_c(const FwdArgs &a) {
  constexpr int MAX_CT = (sizeof(T) == 4 && D == 128) ? 1 : (D >= 64 ? 4 : 2);
  const bool short_seqs = a.total_tokens <= 2 * (int64_t)C * a.num_seqs;
  const int max_ct = short_seqs && MAX_CT > 2 ? 2 : MAX_CT;
  const int64_t units = ((int64_t)a.num_seqs * a.num_heads + 7) / 8;
  const int64_t cus = device_cus();
  auto rounds = [&](int ct) { return cus > 0 ? (8 * units * (D / (16 * ct)) + cus - 1) / cus : 1; };
  int ct = 1;
  for (int c = 2; c <= max_ct; c *= 2)
    if (rounds(c) < rounds(ct)) ct = c;
  if (short_seqs) {
    if constexpr (MAX_CT >= 2) {
      if (ct == 2) return launch_inter_ct<T, D, C, 2, 1, false>(a);
    }
    return launch_inter_ct<T, D, C, 1, 1, false>(a);
  }
  if constexpr (MAX_CT >= 4) {
    if (ct == 4) return launch_inter_ct<T, D, C, 4, 3, false>(a);
  }
  if constexpr (MAX_CT >= 2) {
    if (ct == 2) return launch_inter_ct<T, D, C, 2, 3, false>(a);
  }
  // L2 warm-up loads on 16-column slices of long chains (mean sequence
  // length of at least WARM_MIN_CHUNKS chunks)
  constexpr int64_t WARM_MIN_CHUNKS = 128;
  const bool warm = a.total_tokens >= WARM_MIN_CHUNKS * C * (int64_t)a.num_seqs;
  // bf16, d = 128, C = 64: the split-role form (measured on MI355X: the
  // B=1 H=32 T=32768 chain 512 -> 497 us, B=2 H=8 T=2048 25.6 -> 23.3 us,
  // outputs bitwise equal)
  if constexpr (sizeof(T) == 2 && D == 128 && C == 64) {
    if (warm) return launch_inter_split<T, D, C, true>(a);
    return launch_inter_split<T, D, C, false>(a);
  }
  if (warm) return launch_inter_ct<T, D, C, 1, 3, true>(a);
  return launch_inter_ct<T, D, C, 1, 3, false>(a);
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
      case 128: return launch_inter_d<float, 128>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
