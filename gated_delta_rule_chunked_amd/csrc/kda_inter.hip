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
// 32 or 64 columns) and walks that sequence's chunks.  Its four wavefronts split the rows: wave w
// computes token block w of Unew and O and channel blocks w*CBW.. of S, so
// all four SIMDs issue matrix-core work and each wave loads only its quarter
// of W, Qt, P and Ke.  The blocks meet through two tiny LDS exchanges per
// chunk (Unew after its product, S after the update), each a plain lane-for-
// lane copy: the intra-chunk kernel stores W, Qt (channels) and Ke^T, P
// (tokens) with their contraction index in the kperm order of
// kda_common.hpp, in which a 16x16 output tile held by one wave is already
// half of another wave's K-step operand.  The fp32 state stays in registers.
//
// The intra-chunk kernel stores all of these operands fragment-major
// (frag_off / tile_off), so every load below is one contiguous run per wave.
// Loads are the bottleneck of a serial chain: each wave keeps PF chunks of
// its operands in flight (a ring of register buffers, the loop unrolled by
// PF), requesting chunk c + PF right after the last use of chunk c's group.
// The requests are unconditional (chunks past the end re-read the last one)
// and fenced with scheduling barriers so the compiler keeps them in place.
// Workgroups of one (sequence, head) share blockIdx % 8 and therefore one
// XCD and its L2, which serves the same W/Qt/Ke/P rows to all slices.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

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
    f32x4 gv[CBW];  // e^{G_n} of the wave's channel rows
  };
};

// CT: 16-column tiles per workgroup (a slice of 16 CT columns).  The tiles
// share every W, Qt, P and Ke^T fragment a wave loads, so wider slices halve
// the operand bytes per column but lengthen each serial step; the launch
// takes them only where they cut the rounds of workgroups on the GPU.
template <typename T, int D, int C, int PF, int CT>
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

  __shared__ V4 sS[CT][NCB][64];     // S (operand type), one output tile per channel block
  __shared__ V4 sU[CT][2 * KC][64];  // Unew (operand type), one tile per token block

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
        sS[t][cb][lane] = vec4_from_f32<T>(x);
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
      B.gv[j] = *reinterpret_cast<const f32x4 *>(gam + tile * D + 16 * cb + 4 * lg);
    }
  };
  auto load_all = [&](Buf &B, int ci) {
    load_wu(B, ci);
    load_qp(B, ci);
    load_kg(B, ci);
  };

  auto step = [&](Buf &B, int ci) {
    const int nxt = min(ci + PF, nch - 1);
    const int tc = t0 + ci * C;
    const int rows = min(C, len - ci * C);

    // S entering the chunk, as K-step operands over channels, per column tile
    F sb[CT][KD];
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int ks = 0; ks < KD; ++ks)
        sb[t][ks] = join4(sS[t][2 * ks][lane], sS[t][2 * ks + 1][lane]);

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
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          f32x4 acc = S[j][t] * B.gv[j];
#pragma unroll
          for (int ks = 0; ks < KC; ++ks) acc = mma_k32(B.kA[j][ks], ub[t][ks], acc);
          S[j][t] = acc;
          sS[t][cb][lane] = vec4_from_f32<T>(acc);
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
        for (int ks = 0; ks < KD; ++ks) oc = mma_k32(B.qA[ks], sb[t][ks], oc);
#pragma unroll
        for (int ks = 0; ks < KC; ++ks) oc = mma_k32(B.pA[ks], ub[t][ks], oc);
        // read (and convert) before any branch: matrix-core results are read
        // only in straight-line code after the instructions that produce them;
        // "+ 0" makes it a real VALU read also when T is fp32
        ov[t] = vec4_from_f32<T>(oc + 0.f);
      }
      T *op = o + (int64_t)(tc + 16 * rb + 4 * lg) * rs + (int64_t)h * D + col0 + lr;
      if (rows == C) {
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
    __builtin_amdgcn_sched_barrier(0);
    load_qp(B, nxt);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  };

  static_assert(PF == 3, "the chunk loop below is unrolled for three buffers");
  Buf B0, B1, B2;
  if (nch > 0) {
    load_all(B0, 0);
    load_all(B1, min(1, nch - 1));
    load_all(B2, min(2, nch - 1));
  }
  for (int ci = 0; ci < nch; ci += 3) {
    step(B0, ci);
    if (ci + 1 < nch) step(B1, ci + 1);
    if (ci + 2 < nch) step(B2, ci + 2);
  }

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

template <typename T, int D, int C, int CT>
static hipError_t launch_inter_ct(const FwdArgs &a) {
  constexpr int NS = D / (16 * CT);
  const int pairs = a.num_seqs * a.num_heads;
  const int units = (pairs + 7) / 8;
  const dim3 grid((unsigned)(8 * units * NS));
  char *ws = a.ws;
  hipLaunchKernelGGL((inter_chunk_kernel<T, D, C, 3, CT>), grid, dim3(256), 0, a.stream,
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
template <typename T, int D, int C>
static hipError_t launch_inter_c(const FwdArgs &a) {
  constexpr int MAX_CT = (sizeof(T) == 4 && D == 128) ? 1 : (D >= 64 ? 4 : 2);
  const int64_t units = ((int64_t)a.num_seqs * a.num_heads + 7) / 8;
  const int64_t cus = device_cus();
  auto rounds = [&](int ct) { return cus > 0 ? (8 * units * (D / (16 * ct)) + cus - 1) / cus : 1; };
  int ct = 1;
  for (int c = 2; c <= MAX_CT; c *= 2)
    if (rounds(c) < rounds(ct)) ct = c;
  if constexpr (MAX_CT >= 4) {
    if (ct == 4) return launch_inter_ct<T, D, C, 4>(a);
  }
  if constexpr (MAX_CT >= 2) {
    if (ct == 2) return launch_inter_ct<T, D, C, 2>(a);
  }
  return launch_inter_ct<T, D, C, 1>(a);
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
