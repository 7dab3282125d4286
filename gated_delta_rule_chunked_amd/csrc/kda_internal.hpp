// kda_internal.hpp -- host-side plumbing shared by the C ABI and the kernel
// launchers: the prefill workspace layout and the launcher entry points.
#pragma once

#include <atomic>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Prefill workspace layout.  Per-chunk products are stored per (chunk, head)
// tile, tile index = chunk * H + head, so that every tile is one contiguous
// block; chunk ids enumerate the chunks of sequence 0, then sequence 1, ...
//   seq_first   int  [num_seqs]      first chunk id of each sequence
//   chunk_tab   int4 [max_chunks]    (sequence, first token, rows, 0) per chunk
//                                    id, rows = 0 past the last chunk (packed
//                                    sequences; built once per call)
//   qt          elem [tiles][C][D]   Q * exp(G)
//   w           elem [tiles][C][D]   WY factor W = T Diag(beta) (K * exp(G))
//   ut          elem [tiles][D][C]   WY factor U = T Diag(beta) V, transposed
//   ket         elem [tiles][D][CK]  K * exp(G_last - G), transposed
//   p           elem [tiles][C][CK]  lower-triangular (Q*exp(G)) (K*exp(-G))^T
//   gam         fp32 [tiles][D]      exp(G_last), the chunk's total decay
// CK = max(C, 32) is the token extent padded to one 32-wide matrix-core
// K-step (the padding columns are zero).  The contraction index of qt and w
// (channels) and of ket and p (tokens) is taken in the kperm order of
// kda_common.hpp, the order in which the inter-chunk kernel holds the state
// and the corrected values in registers, and every tile is stored
// fragment-major (frag_off / tile_off in kda_common.hpp) so that the
// inter-chunk kernel reads it with contiguous loads.
struct FwdLayout {
  int64_t max_chunks = 0;
  int64_t tiles = 0;
  size_t seq_first = 0, chunk_tab = 0, qt = 0, w = 0, ut = 0, ket = 0, p = 0, gam = 0,
         total = 0;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// max_chunks: chunk count bound valid for any split of T tokens into N
// sequences (sum of ceil(len_i / C) <= (T + N (C - 1)) / C).
inline FwdLayout fwd_layout(int64_t T, int64_t N, int64_t H, int64_t D,
                            int64_t C, size_t elem) {
  FwdLayout L;
  const int64_t CK = C < 32 ? 32 : C;
  L.max_chunks = (T + N * (C - 1)) / C;
  L.tiles = L.max_chunks * H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  };
  L.seq_first = take(sizeof(int) * (size_t)N);
  L.chunk_tab = take(16 * (size_t)L.max_chunks);
  L.qt = take(elem * (size_t)(L.tiles * C * D));
  L.w = take(elem * (size_t)(L.tiles * C * D));
  L.ut = take(elem * (size_t)(L.tiles * D * C));
  L.ket = take(elem * (size_t)(L.tiles * D * CK));
  L.p = take(elem * (size_t)(L.tiles * C * CK));
  L.gam = take(sizeof(float) * (size_t)(L.tiles * D));
  L.total = off;
  return L;
}

// kda_options (kda.h) resolved on the host.  Input-side fusion: the gate
// function (0 = g given, 1 = softplus gate, 2 = sigmoid gate), A per head
// (softplus gate), g_min (sigmoid gate), the q/k normalisation and
// beta-logit flags.  Serving: state slots.  Output epilogue: RMSNorm weight
// (nullptr = off), output gate input and epsilon.
struct OptArgs {
  int gate = KDA_GATE_LOG_ALPHA;
  const float *gate_A = nullptr;
  float gate_min = 0.f;
  int l2norm_qk = 0, beta_logits = 0;
  const int *slots = nullptr;  // state slot per sequence, or nullptr
  int num_slots = 0;
  const float *norm_w = nullptr;
  const void *out_gate = nullptr;
  float norm_eps = 0.f;
  int heads = 0;  // decode: heads per sequence, to find A of state p
  int *flags = nullptr;  // KDA_FLAG_* bits are ORed in here, or nullptr
  int check = 0;         // nonzero: cu_seqlens was validated into flags first
};

// With OptArgs::check, every prefill kernel returns at once when the
// validation kernel has flagged cu_seqlens (read after a kernel boundary).
__device__ inline bool inputs_rejected(const OptArgs &in) {
  return in.check && (*in.flags & KDA_FLAG_BAD_CU_SEQLENS) != 0;
}

// Arguments common to the two prefill launches.
struct FwdArgs {
  const void *q, *k, *v;
  const void *gate;        // g (fp32) or the gate input z (operand type)
  const float *beta;
  OptArgs in;
  const int *cu_seqlens;  // device, or nullptr for equal lengths
  const int4 *chunk_tab;  // in the workspace when cu_seqlens is set, else nullptr
  int num_seqs, num_heads, d, chunk;
  int64_t total_tokens;
  int seq_len;            // equal-length sequences: tokens per sequence
  int64_t grid_chunks;    // chunk ids to launch (exact when equal lengths)
  const float *s0;
  float *s_final;
  void *o;
  char *ws;
  FwdLayout lay;
  hipStream_t stream;
};

// Backward workspace (kda_bwd_chunked), fp32, per (chunk, head) tile: the
// recomputed chunk factors (row-major [C][D] or [C][C]), the chunk start
// state and the gradient of the state after the chunk ([D][D]; bf16 in the
// first half of their slots for bf16 inputs with C >= 32), the
// gradient of U - W S ([C][D]) and the per-tile scratch of the gradient
// kernel; seq_first [num_seqs] as in the forward.
struct BwdLayout {
  int64_t tiles = 0;
  int64_t scratch_per_tile = 0;  // floats
  int64_t max_chunks = 0;
  size_t seq_first = 0, chunk_tab = 0, kt = 0, kh = 0, qt = 0, ke = 0, w = 0, u = 0, vr = 0,
         gc = 0,
         tm = 0, pm = 0, mm = 0, gam = 0, bt = 0, px = 0, qy = 0, sc = 0, dse = 0, dun = 0,
         scratch = 0, total = 0;
};

inline BwdLayout bwd_layout(int64_t T, int64_t N, int64_t H, int64_t D, int64_t C) {
  BwdLayout L;
  L.max_chunks = (T + N * (C - 1)) / C;
  L.tiles = L.max_chunks * H;
  L.scratch_per_tile = 9 * C * D + 4 * C * C + D;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  };
  const size_t f = sizeof(float), t = (size_t)L.tiles;
  L.seq_first = take(sizeof(int) * (size_t)N);
  L.chunk_tab = take(16 * (size_t)L.max_chunks);
  L.kt = take(f * t * C * D);
  L.kh = take(f * t * C * D);
  L.qt = take(f * t * C * D);
  L.ke = take(f * t * C * D);
  L.w = take(f * t * C * D);
  L.u = take(f * t * C * D);
  L.vr = take(f * t * C * D);
  L.gc = take(f * t * C * D);
  L.tm = take(f * t * C * C);
  L.pm = take(f * t * C * C);
  L.mm = take(f * t * C * C);
  L.gam = take(f * t * D);
  L.bt = take(f * t * C);
  L.px = take(f * t * C * D);  // P^T dO
  L.qy = take(f * t * D * D);  // Qt^T dO
  L.sc = take(f * t * D * D);
  L.dse = take(f * t * D * D);
  L.dun = take(f * t * C * D);
  L.scratch = take(f * t * (size_t)L.scratch_per_tile);
  L.total = off;
  return L;
}

struct BwdArgs {
  const void *q, *k, *v, *d_o;
  const float *g, *beta, *s0, *dsf;
  const int *cu_seqlens;
  const int4 *chunk_tab;  // in the workspace when cu_seqlens is set, else nullptr
  int num_seqs, num_heads, d, chunk, seq_len;
  int64_t grid_chunks;
  void *dq, *dk, *dv;
  float *dg, *dbeta, *ds0;
  char *ws;
  BwdLayout lay;
  hipStream_t stream;
};

// Compute units of the current device (0 if unknown); cached per device.
int device_cus();

// Raises `kernel`'s dynamic-LDS limit to `bytes` on the current device, once
// per device (the limit is a per-device property of a kernel): `done` is the
// launch site's own bit set of devices already raised.  Concurrent first
// calls may both raise it, which is harmless.  Allocates nothing.
inline hipError_t raise_lds_limit(const void *kernel, int bytes,
                                  std::atomic<unsigned long long> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = (dev >= 0 && dev < 64) ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}
hipError_t launch_intra(const FwdArgs &a, kda_dtype dt);
// Builds the chunk table and seq_first of packed sequences from cu [N + 1]
// (one workgroup).  Offsets that break the rules cannot make it write past
// the table or describe chunks outside [0, total); the call's other kernels
// then compute garbage but stay in bounds.  Returns at once when check_inputs
// has flagged cu (in.check).
hipError_t launch_chunk_table(const int *cu, int N, int64_t total, int C, int64_t max_chunks,
                              int4 *tab, int *seq_first, const OptArgs &in, hipStream_t stream);
// Validates cu_seqlens [N + 1] (cu[0] = 0, non-decreasing, cu[N] = total) and
// ORs KDA_FLAG_BAD_CU_SEQLENS into *flags when it fails.
hipError_t launch_check_cu(const int *cu, int N, int64_t total, int *flags, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &a, kda_dtype dt);
hipError_t launch_inter(const FwdArgs &a, kda_dtype dt);
// In place on o [rows, d]: o <- o / sqrt(mean(o^2) + eps) * w * sigmoid(z).
hipError_t launch_out_epilogue(void *o, const OptArgs &in, int64_t rows, int d,
                               kda_dtype dt, hipStream_t stream);
hipError_t launch_decode(const void *q, const void *k, const void *v,
                         const void *gate, const float *beta, const OptArgs &in,
                         float *state, void *o, int batch, int heads, int d,
                         kda_dtype dt, hipStream_t stream);

}  // namespace kda
