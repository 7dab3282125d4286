// kda_decode.hip -- one recurrent KDA step for a batch of fp32 states.
//
// Per (sequence, head) with state S (d x d, rows = key channels):
//   S' = Diag(alpha) S            forget, one rate per key channel
//   u  = beta (v - S'^T k)        delta-rule correction
//   o  = S'^T q + (k . q) u       read-out of the updated state
//   S  = S' + k u^T               erase + write
// (mkdocs.reaper.mx "Attention lineaire et recurrence", section "Kimi Delta
// Attention = les trois remedes combines": forget, erase, write; docsaid.org
// "Kimi Linear", section "KDA : une decroissance propre a chaque canal".)
// The two reductions only need S^T (alpha * k) and S^T (alpha * q), so each
// state is streamed through registers once: one coalesced 16-byte read and
// one 16-byte write per four values.  Decode is bound by HBM bandwidth
// (about one flop per byte).
//
// The state is streamed with nontemporal loads and stores: it is touched
// once per step and would only evict other data from the caches (measured
// about 7% faster on MI355X than plain accesses for 256 x 32 states).
//
// Block = one state.  Thread t owns float4 column group t % (d/4) and the
// RPT consecutive rows from (t / (d/4)) * RPT, so its slices of k, q and the
// gate are a few vector loads, issued ahead of the state rows.  Column sums
// are reduced over the lanes of a wavefront with cross-lane shuffles and over
// wavefronts through LDS.
//
// Occupancy.  For d = 128 and a batch of several rounds of the GPU, each
// workgroup also reserves LDS that it does not use, so that a CU holds two
// workgroups (eight wavefronts, two states streaming) instead of the three
// its registers would allow.  Measured on MI355X for 256 x 32 states: two per
// CU streams about 6.1 TB/s, three about 5.5 and one about 5.4; the fewer
// states are in flight, the fewer DRAM rows the CU's requests spread over,
// until too few requests are left in flight to cover the latency.
//
// Input-side fusion (kda_options): with RAW the gate input is z and the gate
// function gives g per key channel.  With l2norm_qk, q and k enter the step
// only through S^T (alpha k), S^T (alpha q), k . q and k u^T, so their norms
// are reduced alongside k . q and applied as scalar factors.  The output
// epilogue (RMSNorm over the row, output gate) runs on the fp32 row held by
// the first d/4 lanes before it is rounded and stored.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <typename T, int D, int NT, bool RAW>
__global__ __launch_bounds__(NT) void decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const void *__restrict__ gate, const float *__restrict__ beta, const OptArgs in,
    float *__restrict__ state, T *__restrict__ o) {
  constexpr int NCQ = D / 4;         // float4 column groups
  constexpr int NRG = NT / NCQ;      // row groups
  constexpr int RPT = D / NRG;       // rows per thread
  constexpr int NW = NT / 64;        // wavefronts
  static_assert(NT % 64 == 0 && 64 % NCQ == 0 && D % NRG == 0 && RPT % 4 == 0,
                "decode shape");

  __shared__ f32x4 s_x[NW][NCQ];
  __shared__ f32x4 s_y[NW][NCQ];
  __shared__ float s_kq[NW], s_kk[NW], s_qq[NW];

  const int64_t p = blockIdx.x;
  const int tid = threadIdx.x;
  const int cq = tid % NCQ, rg = tid / NCQ;
  int64_t sp = p;  // state of (sequence, head) p: row p, or its slot of the pool
  if (in.slots) {
    const int64_t b = p / in.heads;
    const int sl = in.slots[b];
    if (sl < 0 || sl >= in.num_slots) {  // padding: o = 0, no state touched
      if (rg == 0) store4_f32<T>(o + p * D + 4 * cq, zero4());
      return;
    }
    sp = (int64_t)sl * in.heads + (p - b * in.heads);
  }
  float *S = state + sp * D * D;
  const T *qp = q + p * D;
  const T *kp = k + p * D;
  const float eA = (RAW && in.gate == KDA_GATE_SOFTPLUS) ? __expf(in.gate_A[p % in.heads]) : 0.f;

  const int r0 = rg * RPT;  // first row of this thread
  float kr[RPT], qr[RPT], gr[RPT];
#pragma unroll
  for (int j = 0; j < RPT / 4; ++j) {
    const f32x4 k4 = to_f32x4(load4<T>(kp + r0 + 4 * j));
    const f32x4 q4 = to_f32x4(load4<T>(qp + r0 + 4 * j));
    f32x4 g4;
    if constexpr (RAW) {
      const f32x4 z4 = to_f32x4(load4<T>(reinterpret_cast<const T *>(gate) + p * D + r0 + 4 * j));
      g4 = in.gate == KDA_GATE_SOFTPLUS ? gate_softplus(z4, eA) : gate_sigmoid(z4, in.gate_min);
    } else {
      g4 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(gate) + p * D + r0 +
                                              4 * j);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kr[4 * j + e] = k4[e];
      qr[4 * j + e] = q4[e];
      gr[4 * j + e] = g4[e];
    }
  }
  f32x4 Sv[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    Sv[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (r0 + i) * D + 4 * cq));
  float a[RPT];
  f32x4 x = zero4(), y = zero4();
  float kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    a[i] = __expf(gr[i]);
    kq += kr[i] * qr[i];
    kk += kr[i] * kr[i];
    qq += qr[i] * qr[i];
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    x += Sv[i] * (a[i] * kr[i]);
    y += Sv[i] * (a[i] * qr[i]);
  }
  // reduce over the row groups of this wavefront (lanes cq + NCQ * m)
#pragma unroll
  for (int off = NCQ; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] += __shfl_xor(x[e], off);
      y[e] += __shfl_xor(y[e], off);
    }
    kq += __shfl_xor(kq, off);
    kk += __shfl_xor(kk, off);
    qq += __shfl_xor(qq, off);
  }
  const int wave = tid >> 6, lane = tid & 63;
  if (lane < NCQ) {
    s_x[wave][lane] = x;
    s_y[wave][lane] = y;
  }
  // kq: each row group summed its own rows and the shuffles added the row
  // groups of this wave, so any lane holds the wave's part.
  if (lane == 0) {
    s_kq[wave] = kq;
    s_kk[wave] = kk;
    s_qq[wave] = qq;
  }
  __syncthreads();
  f32x4 xs = zero4(), ys = zero4();
  float kqs = 0.f, kks = 0.f, qqs = 0.f;
#pragma unroll
  for (int wv = 0; wv < NW; ++wv) {
    xs += s_x[wv][cq];
    ys += s_y[wv][cq];
    kqs += s_kq[wv];
    kks += s_kk[wv];
    qqs += s_qq[wv];
  }
  float rk = 1.f;  // k <- rk k, q <- rq q
  if (in.l2norm_qk) {
    rk = rsqrtf(kks + 1e-6f);
    const float rq = rsqrtf(qqs + 1e-6f);
    xs *= rk;
    ys *= rq;
    kqs *= rk * rq;
  }
  const float b = in.beta_logits ? sigmoid(beta[p]) : beta[p];
  f32x4 vv;
  {
    const T *vp = v + p * D + 4 * cq;
    vv = f32x4{to_f32(vp[0]), to_f32(vp[1]), to_f32(vp[2]), to_f32(vp[3])};
  }
  const f32x4 u = b * (vv - xs);
  if (rg == 0) {  // lanes 0 .. NCQ-1 of wave 0 hold the output row
    f32x4 ov = ys + kqs * u;
    if (in.norm_w) {  // output epilogue on the fp32 row: RMSNorm, gate
      const float ss = group_sum<NCQ>(ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] +
                                      ov[3] * ov[3]);
      ov *= rsqrtf(ss * (1.f / D) + in.norm_eps);
      ov *= *reinterpret_cast<const f32x4 *>(in.norm_w + 4 * cq);
      if (in.out_gate) {
        const f32x4 zo = to_f32x4(load4<T>(reinterpret_cast<const T *>(in.out_gate) +
                                           p * D + 4 * cq));
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] *= sigmoid(zo[e]);
      }
    }
    store4_f32<T>(o + p * D + 4 * cq, ov);
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    __builtin_nontemporal_store(a[i] * Sv[i] + (rk * kr[i]) * u,
                                reinterpret_cast<f32x4 *>(S + (r0 + i) * D + 4 * cq));
}

// LDS that a d = 128 workgroup reserves without using it: with the kernel's
// own 4 KiB, three workgroups would need more than a CU's 160 KiB, two fit.
constexpr unsigned kDecodeLdsReserve = 56 * 1024;

template <typename T, int D, int NT>
static void launch_decode_k(const void *q, const void *k, const void *v, const void *gate,
                            const float *beta, const OptArgs &in, float *state, void *o,
                            int pairs, hipStream_t s) {
  const T *qq = reinterpret_cast<const T *>(q);
  const T *kk = reinterpret_cast<const T *>(k);
  const T *vv = reinterpret_cast<const T *>(v);
  T *oo = reinterpret_cast<T *>(o);
  // two workgroups per CU once the batch takes several rounds of the GPU;
  // a smaller batch keeps every state in flight at once
  const int cus = device_cus();
  const unsigned lds = (D == 128 && cus > 0 && pairs >= 4 * cus) ? kDecodeLdsReserve : 0;
  if (in.gate == KDA_GATE_LOG_ALPHA)
    hipLaunchKernelGGL((decode_kernel<T, D, NT, false>), dim3(pairs), dim3(NT), lds, s, qq, kk,
                       vv, gate, beta, in, state, oo);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, NT, true>), dim3(pairs), dim3(NT), lds, s, qq, kk,
                       vv, gate, beta, in, state, oo);
}

template <typename T>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v,
                                  const void *gate, const float *beta, const OptArgs &in,
                                  float *state, void *o, int pairs, int d, hipStream_t s) {
  switch (d) {
    case 32: launch_decode_k<T, 32, 64>(q, k, v, gate, beta, in, state, o, pairs, s); break;
    case 64: launch_decode_k<T, 64, 256>(q, k, v, gate, beta, in, state, o, pairs, s); break;
    case 128: launch_decode_k<T, 128, 256>(q, k, v, gate, beta, in, state, o, pairs, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const void *q, const void *k, const void *v, const void *gate,
                         const float *beta, const OptArgs &in, float *state, void *o,
                         int batch, int heads, int d, kda_dtype dt, hipStream_t stream) {
  const int pairs = batch * heads;
  OptArgs ia = in;
  ia.heads = heads;
  if (dt == KDA_DTYPE_BF16)
    return launch_decode_t<bf16>(q, k, v, gate, beta, ia, state, o, pairs, d, stream);
  return launch_decode_t<float>(q, k, v, gate, beta, ia, state, o, pairs, d, stream);
}

}  // namespace kda
