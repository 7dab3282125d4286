// kda_intra.hip -- intra-chunk kernel: decay-scaled blocks, UT transform and
// WY factors for one (chunk, head) tile.
//
// For a chunk of n <= C tokens with chunk-local cumulative log-decay G
// (rows = tokens, columns = key channels), the token-by-token delta updates
// of the chunk are packed into dense factors (fr.news.hada.io Kimi Linear
// summary, section "Algorithme parallele par chunks": WY representation,
// UT transform, row-by-row forward substitution, intra-chunk work on the
// matrix units; section "Un volume de calcul reduit": both low-rank vectors
// are tied to k, so only two chunk matrices are needed):
//
//   Qt = Q * e^G,  Kt = K * e^G,  Kh = K * e^-G,  Ke = K * e^(G_n - G)
//   A  = strictly_lower(Diag(beta) Kt Kh^T)       (decay-scaled K K^T)
//   P  = lower_with_diagonal(Qt Kh^T)             (decay-scaled Q K^T)
//   T  = (I + A)^-1                               (forward substitution)
//   W  = T Diag(beta) Kt,   U = T Diag(beta) V    (WY factors)
//
// (* = per-channel product.)  These follow from unrolling the recurrence
// over the chunk; the inter-chunk kernel then uses U - W S, Qt S + P(U - W S)
// and e^(G_n) S + Ke^T (U - W S).  The chunk-start reference of Kh requires
// G_n > -80 per channel (exp(80) is far inside fp32/bf16 range), the bound
// quoted in mkdocs.reaper.mx, section "Le piege numerique de la decroissance
// cumulee".
//
// One workgroup of 4 wavefronts per tile.  Phases (barrier-separated):
//  1. elementwise scaling (fp32 exp), 16-byte loads, operands to LDS
//  2. A and P tiles on the matrix cores (16x16 output tiles, K = d)
//  3. T in LDS, fp32: 16x16 diagonal blocks by forward substitution (one
//     wave per block), then the off-diagonal blocks block-row by block-row,
//     T_ij = -T_ii sum_m A_im T_mj, on fp32 MFMA
//  4. W and U on the matrix cores (K = tokens), T rounded to the operand type
//  5. Ke written transposed through LDS
// Qt, W (channels), Ke^T and P (tokens) are stored with their contraction
// index in kperm order (kda_common.hpp) for the inter-chunk kernel, which
// also receives exp(G_last) per channel.
// LDS is reused between phases: the row-major Qt/Kt/Kh copies of phases 1-2
// become T and the transposed Diag(beta)Kt, Diag(beta)V copies of phase 4.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <typename T, int D, int C>
struct IntraCfg {
  static constexpr int NRB = C / 16;              // 16-row blocks of the chunk
  static constexpr int NCB = D / 16;              // 16-col blocks of a head
  static constexpr int CK = C < 32 ? 32 : C;      // token extent per K-step
  static constexpr int PAD = 16 / (int)sizeof(T); // 16-byte row padding
  static constexpr int LDR = D + PAD;             // [C][D] row stride
  static constexpr int LDT = CK + PAD;            // [D][CK] row stride
  static constexpr int LDA = CK + 4;              // fp32 [C][CK] row stride
  static constexpr int GPR = D / 8;               // threads per row, phase 1
  static constexpr int RPP = 256 / GPR;           // rows per pass
  static constexpr int NPASS = (C + RPP - 1) / RPP;
  static constexpr int BYTES_ROW = C * LDR * (int)sizeof(T);
  static constexpr int BYTES_TR = D * LDT * (int)sizeof(T);
  static constexpr int BYTES_X = (2 * BYTES_ROW > 2 * BYTES_TR) ? 2 * BYTES_ROW : 2 * BYTES_TR;
  static constexpr int BYTES_A = C * LDA * 4;
  static constexpr int BYTES_Y = (BYTES_ROW > BYTES_A) ? BYTES_ROW : BYTES_A;
  static constexpr int LDS_BYTES = BYTES_X + BYTES_Y + C * 4;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(C % 16 == 0 && D % 32 == 0, "tile shape");
};

template <typename T, int D, int C>
__global__ __launch_bounds__(256) void intra_chunk_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ gc, const float *__restrict__ beta,
    const int4 *__restrict__ chunk_info, int H, T *__restrict__ qt_out,
    T *__restrict__ w_out, T *__restrict__ ut_out, T *__restrict__ ket_out,
    T *__restrict__ p_out, float *__restrict__ gam_out) {
  using Cfg = IntraCfg<T, D, C>;
  constexpr int NRB = Cfg::NRB, NCB = Cfg::NCB, CK = Cfg::CK;
  constexpr int LDR = Cfg::LDR, LDT = Cfg::LDT, LDA = Cfg::LDA;
  constexpr int GPR = Cfg::GPR, RPP = Cfg::RPP, NPASS = Cfg::NPASS;

  extern __shared__ __align__(16) char smem[];
  T *sK = reinterpret_cast<T *>(smem);                       // [C][LDR]
  T *sKh = reinterpret_cast<T *>(smem + Cfg::BYTES_ROW);     // [C][LDR]
  T *sKbT = reinterpret_cast<T *>(smem);                     // [D][LDT] (later)
  T *sVbT = reinterpret_cast<T *>(smem + Cfg::BYTES_TR);     // [D][LDT] (later)
  T *sQ = reinterpret_cast<T *>(smem + Cfg::BYTES_X);        // [C][LDR]
  float *sT = reinterpret_cast<float *>(smem + Cfg::BYTES_X);  // [C][LDA] (later)
  float *sBeta = reinterpret_cast<float *>(smem + Cfg::BYTES_X + Cfg::BYTES_Y);

  const int c = blockIdx.x, h = blockIdx.y;
  const int4 info = chunk_info[c];
  const int t0 = info.y, n = info.z;
  if (n == 0) return;
  const int64_t tile = (int64_t)c * H + h;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t rs = (int64_t)H * D;  // token stride of [T, H, D] tensors
  const int64_t base = (int64_t)t0 * rs + (int64_t)h * D;

  // ---------------- phase 1: elementwise scaling ----------------
  const int ch0 = (tid % GPR) * 8;
  float gl[8];
  {
    const float *p = gc + base + (int64_t)(n - 1) * rs + ch0;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    gl[0] = a[0]; gl[1] = a[1]; gl[2] = a[2]; gl[3] = a[3];
    gl[4] = b[0]; gl[5] = b[1]; gl[6] = b[2]; gl[7] = b[3];
  }
  if (tid < GPR) {
    float *gp = gam_out + tile * D + ch0;
    *reinterpret_cast<f32x4 *>(gp) =
        f32x4{__expf(gl[0]), __expf(gl[1]), __expf(gl[2]), __expf(gl[3])};
    *reinterpret_cast<f32x4 *>(gp + 4) =
        f32x4{__expf(gl[4]), __expf(gl[5]), __expf(gl[6]), __expf(gl[7])};
  }
  T kb_reg[NPASS][8], vb_reg[NPASS][8], ke_reg[NPASS][8];
  T *qt_tile = qt_out + tile * (C * D);
#pragma unroll
  for (int j = 0; j < NPASS; ++j) {
    const int r = j * RPP + tid / GPR;
    if (r >= C) continue;
    float qt[8], kt[8], kh[8], kbv[8], vbv[8], kev[8];
    if (r < n) {
      const int64_t off = base + (int64_t)r * rs + ch0;
      float G[8], qv[8], kv[8], vv[8];
      load8_f32<float>(gc + off, G);
      load8_f32<T>(q + off, qv);
      load8_f32<T>(k + off, kv);
      load8_f32<T>(v + off, vv);
      const float br = beta[(int64_t)(t0 + r) * H + h];
      if (tid % GPR == 0) sBeta[r] = br;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float eg = __expf(G[e]);
        const float eng = __expf(-G[e]);
        const float ee = __expf(gl[e] - G[e]);
        qt[e] = qv[e] * eg;
        kt[e] = kv[e] * eg;
        kh[e] = kv[e] * eng;
        kbv[e] = br * kt[e];
        vbv[e] = br * vv[e];
        kev[e] = kv[e] * ee;
      }
    } else {
      if (tid % GPR == 0) sBeta[r] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) qt[e] = kt[e] = kh[e] = kbv[e] = vbv[e] = kev[e] = 0.f;
    }
    store8<T>(sQ + r * LDR + ch0, qt);
    store8<T>(sK + r * LDR + ch0, kt);
    store8<T>(sKh + r * LDR + ch0, kh);
    // channels ch0..ch0+3 and ch0+4..ch0+7 are two contiguous runs in kperm order
    store4_f32<T>(qt_tile + frag_off(r, kperm_pos(ch0), D), f32x4{qt[0], qt[1], qt[2], qt[3]});
    store4_f32<T>(qt_tile + frag_off(r, kperm_pos(ch0 + 4), D),
                  f32x4{qt[4], qt[5], qt[6], qt[7]});
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kb_reg[j][e] = from_f32<T>(kbv[e]);
      vb_reg[j][e] = from_f32<T>(vbv[e]);
      ke_reg[j][e] = from_f32<T>(kev[e]);
    }
  }
  __syncthreads();

  // ---------------- phase 2: A and P on the matrix cores ----------------
  constexpr int NLOW = NRB * (NRB + 1) / 2;  // lower tiles incl. diagonal
  constexpr int NAW = (NLOW + 3) / 4;        // per wave
  f32x4 a_keep[NAW];
  int a_rb[NAW], a_cb[NAW];
  T *p_tile = p_out + tile * (C * CK);
#pragma unroll
  for (int j = 0; j < NAW; ++j) {
    a_rb[j] = -1;
    a_cb[j] = 0;
    a_keep[j] = zero4();
    const int idx = wave + 4 * j;
    if (idx >= NLOW) continue;
    int rb = 0, rem = idx;
    while (rem > rb) { rem -= rb + 1; ++rb; }
    const int cb = rem;
    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int kk = 32 * ks + 8 * lg;
      const auto bk = load8<T>(sKh + (16 * cb + lr) * LDR + kk);
      const auto ak = load8<T>(sK + (16 * rb + lr) * LDR + kk);
      const auto aq = load8<T>(sQ + (16 * rb + lr) * LDR + kk);
      accA = mma_k32(ak, bk, accA);
      accP = mma_k32(aq, bk, accP);
    }
    const int col = 16 * cb + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rb + 4 * lg + i;
      accA[i] = (col < row) ? sBeta[row] * accA[i] : 0.f;
      p_tile[frag_off(row, kperm_pos(col), CK)] = from_f32<T>((col <= row) ? accP[i] : 0.f);
    }
    a_keep[j] = accA;
    a_rb[j] = rb;
    a_cb[j] = cb;
  }
  // zero the strictly-upper tiles of P and its padding columns
  for (int e = tid; e < C * CK; e += 256) {
    const int row = e / CK, col = kperm_idx(e % CK);
    if (col >= C || (col / 16) > (row / 16)) p_tile[frag_off(row, e % CK, CK)] = from_f32<T>(0.f);
  }
  __syncthreads();

  // ---------------- phase 3a: A into sT, transposed operands ----------------
  for (int e = tid; e < C * LDA; e += 256) sT[e] = 0.f;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NAW; ++j) {
    if (a_rb[j] < 0) continue;
    const int col = 16 * a_cb[j] + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) sT[(16 * a_rb[j] + 4 * lg + i) * LDA + col] = a_keep[j][i];
  }
#pragma unroll
  for (int j = 0; j < NPASS; ++j) {
    const int r = j * RPP + tid / GPR;
    if (r >= C) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sKbT[(ch0 + e) * LDT + r] = kb_reg[j][e];
      sVbT[(ch0 + e) * LDT + r] = vb_reg[j][e];
    }
  }
  if (CK > C) {  // zero the padding tokens of the transposed operands
    for (int e = tid; e < D * (CK - C); e += 256) {
      const int ch = e / (CK - C), r = C + e % (CK - C);
      sKbT[ch * LDT + r] = from_f32<T>(0.f);
      sVbT[ch * LDT + r] = from_f32<T>(0.f);
    }
  }
  __syncthreads();

  // ---------------- phase 3b: diagonal blocks, forward substitution -------
  if (wave < NRB && lane < 16) {
    const int b0 = 16 * wave;
    const int jcol = lane;
    float tcol[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) tcol[m] = (m == jcol) ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s += sT[(b0 + r) * LDA + b0 + m] * tcol[m];
      if (jcol < r) tcol[r] = -s;
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) sT[(b0 + m) * LDA + b0 + jcol] = tcol[m];
  }
  __syncthreads();

  // ---------------- phase 3c: off-diagonal blocks -------------------------
  // T_ij = -T_ii X,  X = sum_{m=j}^{i-1} A_im T_mj, for block row i, j < i.
#pragma unroll
  for (int bi = 1; bi < NRB; ++bi) {
    f32x4 X = zero4();
    const int bj = wave;
    if (bj < bi) {
      for (int m = bj; m < bi; ++m) {
        const f32x4 af = *reinterpret_cast<const f32x4 *>(
            sT + (16 * bi + lr) * LDA + 16 * m + 4 * lg);
        f32x4 bf;
#pragma unroll
        for (int i = 0; i < 4; ++i) bf[i] = sT[(16 * m + 4 * lg + i) * LDA + 16 * bj + lr];
        X = mma_f32_k16(af, bf, X);
      }
    }
    __syncthreads();
    if (bj < bi) {
      const f32x4 af = *reinterpret_cast<const f32x4 *>(
          sT + (16 * bi + lr) * LDA + 16 * bi + 4 * lg);
      const f32x4 Y = mma_f32_k16(af, X, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) sT[(16 * bi + 4 * lg + i) * LDA + 16 * bj + lr] = -Y[i];
    }
    __syncthreads();
  }

  // ---------------- phase 4: W = T Diag(beta)Kt, U = T Diag(beta)V ---------
  T *w_tile = w_out + tile * (C * D);
  T *ut_tile = ut_out + tile * (D * C);
  constexpr int NWU = 2 * NRB * NCB;
  for (int idx = wave; idx < NWU; idx += 4) {
    const int which = idx / (NRB * NCB);  // 0 = W, 1 = U
    const int rb = (idx % (NRB * NCB)) / NCB;
    const int cb = idx % NCB;
    const T *bsrc = which ? sVbT : sKbT;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < CK / 32; ++ks) {
      if (32 * ks > 16 * rb + 15) break;  // T is lower triangular
      const int kk = 32 * ks + 8 * lg;
      const auto a = frag_from_f32<T>(sT + (16 * rb + lr) * LDA + kk);
      const auto b = load8<T>(bsrc + (16 * cb + lr) * LDT + kk);
      acc = mma_k32(a, b, acc);
    }
    const int col = 16 * cb + lr;
    if (which == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w_tile[frag_off(16 * rb + 4 * lg + i, kperm_pos(col), D)] = from_f32<T>(acc[i]);
    } else {
      store4_f32<T>(ut_tile + tile_off(16 * rb + 4 * lg, col, C), acc);
    }
  }
  __syncthreads();

  // ---------------- phase 5: Ke transposed, through LDS --------------------
  T *sKeT = sKbT;
#pragma unroll
  for (int j = 0; j < NPASS; ++j) {
    const int r = j * RPP + tid / GPR;
    if (r >= C) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) sKeT[(ch0 + e) * LDT + kperm_pos(r)] = ke_reg[j][e];
  }
  if (CK > C) {
    for (int e = tid; e < D * (CK - C); e += 256) {
      const int ch = e / (CK - C), r = C + e % (CK - C);
      sKeT[ch * LDT + kperm_pos(r)] = from_f32<T>(0.f);
    }
  }
  __syncthreads();
  T *ket_tile = ket_out + tile * (D * CK);
  constexpr int V8 = CK / 8;  // 8-element vectors per row
  for (int e = tid; e < D * V8; e += 256) {
    const int ch = e / V8, x = (e % V8) * 8;
    *reinterpret_cast<typename Frag<T>::type *>(ket_tile + frag_off(ch, x, CK)) =
        load8<T>(sKeT + ch * LDT + x);
  }
}

template <typename T, int D, int C>
static hipError_t launch_intra_t(const FwdArgs &a) {
  using Cfg = IntraCfg<T, D, C>;
  auto kern = intra_chunk_kernel<T, D, C>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)a.grid_chunks, (unsigned)a.num_heads);
  char *ws = a.ws;
  hipLaunchKernelGGL(kern, grid, dim3(256), Cfg::LDS_BYTES, a.stream,
                     reinterpret_cast<const T *>(a.q), reinterpret_cast<const T *>(a.k),
                     reinterpret_cast<const T *>(a.v),
                     reinterpret_cast<const float *>(ws + a.lay.gc), a.beta,
                     reinterpret_cast<const int4 *>(ws + a.lay.chunk_info), a.num_heads,
                     reinterpret_cast<T *>(ws + a.lay.qt), reinterpret_cast<T *>(ws + a.lay.w),
                     reinterpret_cast<T *>(ws + a.lay.ut), reinterpret_cast<T *>(ws + a.lay.ket),
                     reinterpret_cast<T *>(ws + a.lay.p), reinterpret_cast<float *>(ws + a.lay.gam));
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_intra_d(const FwdArgs &a) {
  switch (a.chunk) {
    case 16: return launch_intra_t<T, D, 16>(a);
    case 32: return launch_intra_t<T, D, 32>(a);
    case 64: return launch_intra_t<T, D, 64>(a);
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
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
