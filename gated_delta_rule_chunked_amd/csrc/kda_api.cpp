// kda_api.cpp -- the C ABI declared in include/kda.h: host-side argument
// validation, workspace layout and the ordered launches of the prefill
// kernels (intra-chunk -> inter-chunk) and of the decode kernel.  Nothing
// here allocates memory or keeps state; the kernels' launch code keeps, per
// device, only the CU count and which kernels have had their LDS limit raised.
#include <hip/hip_runtime.h>

#include "kda.h"
#include "kda_internal.hpp"

using namespace kda;

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool head_dims_supported(int32_t d_k, int32_t d_v, kda_dtype dtype) {
  if (d_k != d_v) return false;
  if (dtype == KDA_DTYPE_BF16 || dtype == KDA_DTYPE_F32)
    return d_k == 32 || d_k == 64 || d_k == 128;
  return false;
}

size_t elem_size(kda_dtype dt) { return dt == KDA_DTYPE_BF16 ? 2 : 4; }

// Resolves kda_options (NULL = the plain call) into `out`.
kda_status resolve_options(const kda_options *in, OptArgs *out) {
  *out = OptArgs();
  if (in == nullptr) return KDA_SUCCESS;
  if (in->gate != KDA_GATE_LOG_ALPHA && in->gate != KDA_GATE_SOFTPLUS &&
      in->gate != KDA_GATE_SIGMOID)
    return KDA_ERROR_INVALID_VALUE;
  if (in->gate == KDA_GATE_SOFTPLUS && (!in->gate_A || !aligned(in->gate_A, 4)))
    return KDA_ERROR_INVALID_VALUE;
  if (in->gate == KDA_GATE_SIGMOID && !(in->gate_min < 0.f && in->gate_min > -3.0e38f))
    return KDA_ERROR_INVALID_VALUE;  // also rejects NaN
  out->gate = in->gate;
  out->gate_A = in->gate == KDA_GATE_SOFTPLUS ? in->gate_A : nullptr;
  out->gate_min = in->gate == KDA_GATE_SIGMOID ? in->gate_min : 0.f;
  out->l2norm_qk = in->l2norm_qk != 0;
  out->beta_logits = in->beta_logits != 0;
  if (in->state_slots) {
    if (!aligned(in->state_slots, 4) || in->num_slots < 1) return KDA_ERROR_INVALID_VALUE;
    out->slots = in->state_slots;
    out->num_slots = in->num_slots;
  }
  if (in->out_gate && !in->out_norm_weight) return KDA_ERROR_INVALID_VALUE;
  if (in->out_norm_weight) {
    if (!aligned(in->out_norm_weight, 16) || (in->out_gate && !aligned(in->out_gate, 16)))
      return KDA_ERROR_INVALID_VALUE;
    if (!(in->out_norm_eps > 0.f && in->out_norm_eps < 3.0e38f))  // also rejects NaN
      return KDA_ERROR_INVALID_VALUE;
    out->norm_w = in->out_norm_weight;
    out->out_gate = in->out_gate;
    out->norm_eps = in->out_norm_eps;
  }
  if (in->flags && !aligned(in->flags, 4)) return KDA_ERROR_INVALID_VALUE;
  if (in->check_inputs && !in->flags) return KDA_ERROR_INVALID_VALUE;
  out->flags = in->flags;
  out->check = in->check_inputs != 0;
  return KDA_SUCCESS;
}

// Size checks shared by the workspace query and the prefill call.
kda_status check_fwd_sizes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads,
                           int32_t d_k, int32_t d_v, int32_t chunk_size, kda_dtype dtype) {
  if (total_tokens < 0 || num_seqs < 1 || num_heads < 1 || d_k < 1 || d_v < 1 ||
      chunk_size < 1)
    return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERROR_INVALID_VALUE;
  if (!head_dims_supported(d_k, d_v, dtype)) return KDA_ERROR_NOT_SUPPORTED;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return KDA_ERROR_NOT_SUPPORTED;
  // index arithmetic inside the kernels uses 32-bit token and chunk ids
  if (total_tokens > (int64_t)1 << 30 || (int64_t)num_seqs * num_heads > (int64_t)1 << 26)
    return KDA_ERROR_NOT_SUPPORTED;
  const int64_t max_chunks = (total_tokens + (int64_t)num_seqs * (chunk_size - 1)) / chunk_size;
  if (max_chunks > (int64_t)1 << 30 || num_heads > 65535) return KDA_ERROR_NOT_SUPPORTED;
  // one workgroup per (chunk, head) tile on a 1-D grid
  if (max_chunks * num_heads > (int64_t)1 << 22) return KDA_ERROR_NOT_SUPPORTED;
  return KDA_SUCCESS;
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
  switch (s) {
    case KDA_SUCCESS: return "KDA_SUCCESS";
    case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
    case KDA_ERROR_NOT_SUPPORTED: return "KDA_ERROR_NOT_SUPPORTED";
    case KDA_ERROR_LAUNCH_FAILED: return "KDA_ERROR_LAUNCH_FAILED";
    case KDA_ERROR_SCRATCH_TOO_SMALL: return "KDA_ERROR_SCRATCH_TOO_SMALL";
  }
  return "KDA_UNKNOWN_STATUS";
}

int kda_version(void) { return 100; }

size_t kda_fwd_chunked_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                      int32_t num_heads, int32_t d_k, int32_t d_v,
                                      int32_t chunk_size, kda_dtype dtype) {
  if (check_fwd_sizes(total_tokens, num_seqs, num_heads, d_k, d_v, chunk_size, dtype) !=
      KDA_SUCCESS)
    return 0;
  return fwd_layout(total_tokens, num_seqs, num_heads, d_k, chunk_size, elem_size(dtype))
      .total;
}

}  // extern "C"

namespace {

// Validates the prefill arguments and runs the stages selected by `mask`
// (bit s = stage s) in order.
kda_status fwd_run(unsigned mask, const kda_options *options, const void *q, const void *k,
                   const void *v, const void *gate, const float *beta,
                   const int32_t *cu_seqlens,
                   int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k,
                   int32_t d_v, int32_t chunk_size, kda_dtype dtype,
                   const float *initial_state, float *final_state, void *o,
                   void *workspace, size_t workspace_bytes, void *stream) {
  if (mask == 0u || mask > 3u) return KDA_ERROR_INVALID_VALUE;
  OptArgs in;
  kda_status st = resolve_options(options, &in);
  if (st != KDA_SUCCESS) return st;
  st = check_fwd_sizes(total_tokens, num_seqs, num_heads, d_k, d_v, chunk_size, dtype);
  if (st != KDA_SUCCESS) return st;
  if (total_tokens > 0) {
    if (!q || !k || !v || !gate || !beta || !o) return KDA_ERROR_INVALID_VALUE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(gate, 16) || !aligned(beta, 4))
      return KDA_ERROR_INVALID_VALUE;
  }
  if (!cu_seqlens && (total_tokens % num_seqs) != 0) return KDA_ERROR_INVALID_VALUE;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERROR_INVALID_VALUE;
  if ((initial_state && !aligned(initial_state, 16)) ||
      (final_state && !aligned(final_state, 16)))
    return KDA_ERROR_INVALID_VALUE;
  const FwdLayout lay =
      fwd_layout(total_tokens, num_seqs, num_heads, d_k, chunk_size, elem_size(dtype));
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total)
    return KDA_ERROR_INVALID_VALUE;

  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate;
  a.beta = beta;
  a.in = in;
  a.cu_seqlens = cu_seqlens;
  a.chunk_tab = cu_seqlens ? reinterpret_cast<const int4 *>(reinterpret_cast<char *>(workspace) +
                                                            lay.chunk_tab)
                           : nullptr;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.d = d_k;
  a.chunk = chunk_size;
  a.total_tokens = total_tokens;
  a.seq_len = cu_seqlens ? 0 : (int)(total_tokens / num_seqs);
  if (cu_seqlens)
    a.grid_chunks = lay.max_chunks;
  else
    a.grid_chunks = (int64_t)num_seqs * ((a.seq_len + chunk_size - 1) / chunk_size);
  a.s0 = initial_state;
  a.s_final = final_state;
  a.o = o;
  a.ws = reinterpret_cast<char *>(workspace);
  a.lay = lay;
  a.stream = reinterpret_cast<hipStream_t>(stream);

  if (in.check && cu_seqlens &&
      launch_check_cu(cu_seqlens, num_seqs, total_tokens, in.flags, a.stream) != hipSuccess)
    return KDA_ERROR_LAUNCH_FAILED;
  if ((mask & 1u) && cu_seqlens &&
      launch_chunk_table(cu_seqlens, num_seqs, total_tokens, chunk_size, lay.max_chunks,
                         reinterpret_cast<int4 *>(a.ws + lay.chunk_tab),
                         reinterpret_cast<int *>(a.ws + lay.seq_first), in,
                         a.stream) != hipSuccess)
    return KDA_ERROR_LAUNCH_FAILED;
  if ((mask & 1u) && launch_intra(a, dtype) != hipSuccess) return KDA_ERROR_LAUNCH_FAILED;
  if ((mask & 2u) && launch_inter(a, dtype) != hipSuccess) return KDA_ERROR_LAUNCH_FAILED;
  if ((mask & 2u) && in.norm_w && total_tokens > 0 &&
      launch_out_epilogue(o, in, total_tokens * num_heads, d_v, dtype, a.stream) != hipSuccess)
    return KDA_ERROR_LAUNCH_FAILED;
  return KDA_SUCCESS;
}

}  // namespace

extern "C" {

kda_status kda_fwd_chunked(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const int32_t *cu_seqlens, int32_t num_seqs,
                           int64_t total_tokens, int32_t num_heads, int32_t d_k,
                           int32_t d_v, int32_t chunk_size, kda_dtype dtype,
                           const float *initial_state, float *final_state, void *o,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_run(3u, nullptr, q, k, v, log_alpha, beta, cu_seqlens, num_seqs, total_tokens,
                 num_heads, d_k, d_v, chunk_size, dtype, initial_state, final_state, o,
                 workspace, workspace_bytes, stream);
}

kda_status kda_fwd_chunked_stage(kda_fwd_stage stage, const void *q, const void *k,
                                 const void *v, const float *log_alpha, const float *beta,
                                 const int32_t *cu_seqlens, int32_t num_seqs,
                                 int64_t total_tokens, int32_t num_heads, int32_t d_k,
                                 int32_t d_v, int32_t chunk_size, kda_dtype dtype,
                                 const float *initial_state, float *final_state, void *o,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  if (stage != KDA_STAGE_INTRA && stage != KDA_STAGE_INTER) return KDA_ERROR_INVALID_VALUE;
  return fwd_run(1u << (unsigned)stage, nullptr, q, k, v, log_alpha, beta, cu_seqlens,
                 num_seqs, total_tokens, num_heads, d_k, d_v, chunk_size, dtype,
                 initial_state, final_state, o, workspace, workspace_bytes, stream);
}

kda_status kda_fwd_chunked_ex(const kda_options *options, uint32_t stages, const void *q,
                              const void *k, const void *v, const void *gate,
                              const float *beta, const int32_t *cu_seqlens,
                              int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                              int32_t d_k, int32_t d_v, int32_t chunk_size,
                              kda_dtype dtype, const float *initial_state,
                              float *final_state, void *o, void *workspace,
                              size_t workspace_bytes, void *stream) {
  return fwd_run(stages, options, q, k, v, gate, beta, cu_seqlens, num_seqs, total_tokens,
                 num_heads, d_k, d_v, chunk_size, dtype, initial_state, final_state, o,
                 workspace, workspace_bytes, stream);
}

size_t kda_bwd_chunked_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                      int32_t num_heads, int32_t d_k, int32_t d_v,
                                      int32_t chunk_size, kda_dtype dtype) {
  if (check_fwd_sizes(total_tokens, num_seqs, num_heads, d_k, d_v, chunk_size, dtype) !=
      KDA_SUCCESS)
    return 0;
  return bwd_layout(total_tokens, num_seqs, num_heads, d_k, chunk_size).total;
}

kda_status kda_bwd_chunked(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const int32_t *cu_seqlens, int32_t num_seqs,
                           int64_t total_tokens, int32_t num_heads, int32_t d_k,
                           int32_t d_v, int32_t chunk_size, kda_dtype dtype,
                           const float *initial_state, const void *d_o,
                           const float *d_final_state, void *dq, void *dk, void *dv,
                           float *dlog_alpha, float *dbeta, float *d_initial_state,
                           void *workspace, size_t workspace_bytes, void *stream) {
  const kda_status st =
      check_fwd_sizes(total_tokens, num_seqs, num_heads, d_k, d_v, chunk_size, dtype);
  if (st != KDA_SUCCESS) return st;
  if (total_tokens > 0) {
    if (!q || !k || !v || !log_alpha || !beta || !d_o || !dq || !dk || !dv || !dlog_alpha ||
        !dbeta)
      return KDA_ERROR_INVALID_VALUE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_o, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(log_alpha, 16) ||
        !aligned(dlog_alpha, 16) || !aligned(beta, 4) || !aligned(dbeta, 4))
      return KDA_ERROR_INVALID_VALUE;
  }
  if (!cu_seqlens && (total_tokens % num_seqs) != 0) return KDA_ERROR_INVALID_VALUE;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERROR_INVALID_VALUE;
  if ((initial_state && !aligned(initial_state, 16)) ||
      (d_final_state && !aligned(d_final_state, 16)) ||
      (d_initial_state && !aligned(d_initial_state, 16)))
    return KDA_ERROR_INVALID_VALUE;
  const BwdLayout lay = bwd_layout(total_tokens, num_seqs, num_heads, d_k, chunk_size);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total)
    return KDA_ERROR_INVALID_VALUE;
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.d_o = d_o;
  a.g = log_alpha;
  a.beta = beta;
  a.s0 = initial_state;
  a.dsf = d_final_state;
  a.cu_seqlens = cu_seqlens;
  a.chunk_tab = cu_seqlens ? reinterpret_cast<const int4 *>(reinterpret_cast<char *>(workspace) +
                                                            lay.chunk_tab)
                           : nullptr;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.d = d_k;
  a.chunk = chunk_size;
  a.seq_len = cu_seqlens ? 0 : (int)(total_tokens / num_seqs);
  a.grid_chunks = cu_seqlens ? (total_tokens + (int64_t)num_seqs * (chunk_size - 1)) / chunk_size
                             : (int64_t)num_seqs * ((a.seq_len + chunk_size - 1) / chunk_size);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dlog_alpha;
  a.dbeta = dbeta;
  a.ds0 = d_initial_state;
  a.ws = reinterpret_cast<char *>(workspace);
  a.lay = lay;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  if (cu_seqlens &&
      launch_chunk_table(cu_seqlens, num_seqs, total_tokens, chunk_size, lay.max_chunks,
                         reinterpret_cast<int4 *>(a.ws + lay.chunk_tab),
                         reinterpret_cast<int *>(a.ws + lay.seq_first), OptArgs(),
                         a.stream) != hipSuccess)
    return KDA_ERROR_LAUNCH_FAILED;
  if (launch_bwd(a, dtype) != hipSuccess) return KDA_ERROR_LAUNCH_FAILED;
  return KDA_SUCCESS;
}

kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta, float *state,
                           void *o, int32_t batch, int32_t num_heads, int32_t d_k,
                           int32_t d_v, kda_dtype dtype, void *stream) {
  return kda_decode_step_ex(nullptr, q, k, v, log_alpha, beta, state, o, batch, num_heads,
                            d_k, d_v, dtype, stream);
}

kda_status kda_decode_step_ex(const kda_options *options, const void *q, const void *k,
                              const void *v, const void *gate, const float *beta,
                              float *state, void *o, int32_t batch, int32_t num_heads,
                              int32_t d_k, int32_t d_v, kda_dtype dtype, void *stream) {
  OptArgs in;
  const kda_status st = resolve_options(options, &in);
  if (st != KDA_SUCCESS) return st;
  if (batch < 1 || num_heads < 1 || d_k < 1 || d_v < 1) return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERROR_INVALID_VALUE;
  if (d_k != d_v || !(d_k == 32 || d_k == 64 || d_k == 128)) return KDA_ERROR_NOT_SUPPORTED;
  if ((int64_t)batch * num_heads > ((int64_t)1 << 31) - 1) return KDA_ERROR_NOT_SUPPORTED;
  if (!q || !k || !v || !gate || !beta || !state || !o) return KDA_ERROR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(gate, 16) || !aligned(state, 16) || !aligned(beta, 4))
    return KDA_ERROR_INVALID_VALUE;
  if (launch_decode(q, k, v, gate, beta, in, state, o, batch, num_heads, d_k, dtype,
                    reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERROR_LAUNCH_FAILED;
  return KDA_SUCCESS;
}

}  // extern "C"
