/*
 * kda.h -- C ABI of the Kimi Delta Attention (KDA) operator for AMD MI355X
 * (gfx950).
 *
 * KDA is the gated delta rule with one decay per key channel.  For each
 * sequence and head, with a state S of d_k x d_v values (rows = key
 * channels, multiplied from the left):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * (docsaid.org "Kimi Linear -- L'oubli canal par canal", section "KDA : une
 * decroissance propre a chaque canal", second display equation; the
 * read-out is taken on the updated state.)  The decay is passed as its
 * logarithm g = log(alpha) <= 0, per token, head and key channel.  The
 * operator does not normalise q or k and applies no 1/sqrt(d) scale: the
 * layer above L2-normalises q and k and produces beta with a sigmoid and
 * alpha with its gate (same page, section "Les autres pieces").
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, row-major and contiguous.  The
 *     caller owns and allocates every buffer, the workspace included; the
 *     library allocates nothing and may be called from several host
 *     threads on different streams.  Between calls it keeps only what it
 *     reads once per device and kernel: the CU count (which picks the
 *     inter-chunk slice width) and kernel LDS attributes.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *     stream) and return.  Errors raised while the kernels run surface at
 *     the caller's next synchronisation, as for any HIP launch.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     failure nothing is enqueued and the status says why.  Device data
 *     (cu_seqlens contents, tensor values) is never read on the host.
 *   - dtype selects the type of q, k, v and o: KDA_DTYPE_BF16 (bf16
 *     operands on the matrix cores with fp32 accumulation) or
 *     KDA_DTYPE_F32 (fp32 throughout).  log_alpha, beta and the states are
 *     always fp32.
 *   - Supported head sizes: d_k == d_v in {32, 64, 128}, for both
 *     dtypes; other shapes return KDA_ERROR_NOT_SUPPORTED.
 *   - Size limits (KDA_ERROR_NOT_SUPPORTED beyond them): total_tokens <=
 *     2^30, num_seqs * num_heads <= 2^26, num_heads <= 65535 and at most
 *     2^22 (chunk, head) tiles, where a call has at most
 *     (total_tokens + num_seqs * (chunk_size - 1)) / chunk_size chunks.
 *   - No C++ exception crosses this interface.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_SUCCESS = 0,
  KDA_ERROR_INVALID_VALUE = 1, /* null/misaligned pointer, bad size, small workspace */
  KDA_ERROR_NOT_SUPPORTED = 2, /* valid request the library has no kernel for */
  KDA_ERROR_LAUNCH_FAILED = 3, /* the HIP runtime refused a kernel launch */
  KDA_ERROR_SCRATCH_TOO_SMALL = 4 /* kda_fwd_chunked_noalloc: the call needs more
                                     workspace than KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype;

/* Static, human-readable name of a status; never NULL. */
const char *kda_status_string(kda_status status);

/* Library version as major*10000 + minor*100 + patch. */
int kda_version(void);

/*
 * Bytes of device workspace kda_fwd_chunked needs for these sizes (0 if the
 * sizes are invalid or unsupported).  The value depends only on the
 * arguments, never on cu_seqlens contents: for varlen calls it covers the
 * largest chunk count any split of total_tokens into num_seqs sequences can
 * produce.
 */
size_t kda_fwd_chunked_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                      int32_t num_heads, int32_t d_k,
                                      int32_t d_v, int32_t chunk_size,
                                      kda_dtype dtype);

/*
 * Chunked prefill over one or more packed sequences.
 *
 * Splits every sequence into chunks of chunk_size tokens (the last chunk of
 * a sequence may be shorter; chunks never straddle sequences), carries the
 * state from chunk to chunk, and inside a chunk replaces the token-by-token
 * updates with dense products: the decay-scaled K K^T and Q K^T blocks, the
 * UT-transform inverse (I + A)^{-1} of the strictly lower A by forward
 * substitution, and the WY factors W and U (fr.news.hada.io Kimi Linear
 * summary, section "Algorithme parallele par chunks"; mkdocs.reaper.mx
 * "Attention lineaire et recurrence", section "Le calcul par blocs"; the
 * result equals the recurrence up to rounding).
 *
 *   q, k        [total_tokens, H, d_k]  dtype
 *   v           [total_tokens, H, d_v]  dtype
 *   log_alpha   [total_tokens, H, d_k]  fp32, g = log(alpha), finite, <= 0
 *   beta        [total_tokens, H]       fp32, in [0, 1]
 *   cu_seqlens  [num_seqs + 1] int32 device array of sequence offsets
 *               (0 = cu[0] <= cu[1] <= ... <= cu[num_seqs] = total_tokens),
 *               or NULL for num_seqs sequences of total_tokens/num_seqs
 *               tokens each.  Empty sequences are allowed.  Contents that
 *               break these rules are undefined behaviour.
 *   initial_state [num_seqs, H, d_k, d_v] fp32, or NULL for zero states.
 *               May be the same buffer as final_state (updated in place).
 *   final_state [num_seqs, H, d_k, d_v] fp32, or NULL to skip it.  An empty
 *               sequence's final state is its initial state.
 *   o           [total_tokens, H, d_v]  dtype (output)
 *   workspace   device buffer of at least kda_fwd_chunked_workspace_size()
 *               bytes, 256-byte aligned; contents on entry are ignored and
 *               are clobbered.  Calls that share a workspace must be
 *               ordered (same stream or synchronised).
 *   stream      hipStream_t or NULL.
 *
 * Decay range (mkdocs.reaper.mx, section "Le piege numerique de la
 * decroissance cumulee": the chunk form divides by the cumulative decay, and
 * the page bounds it over a 16-token tile).  Chunks whose summed log-decay
 * stays >= -80 in every channel are referenced to the chunk start; a chunk
 * that decays further is referenced per 16-token block, which is exact for
 * any decay as long as every 16-token block's summed log-decay is >= -80 per
 * channel (e^80 is finite in fp32 and bf16).  That block bound is the only
 * precondition: past it outputs may be inf/NaN, and kda_fwd_chunked_ex
 * reports the breach in kda_options.flags (KDA_FLAG_DECAY_RANGE).  Per-token
 * log-decays >= -5 always meet it.
 *
 * q, k, v, o and the states must be 16-byte aligned; log_alpha 16-byte;
 * beta and cu_seqlens 4-byte.  chunk_size must be 16, 32 or 64.
 * total_tokens may be 0 (then q, k, v, log_alpha, beta and o may be NULL).
 */
kda_status kda_fwd_chunked(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const int32_t *cu_seqlens, int32_t num_seqs,
                           int64_t total_tokens, int32_t num_heads,
                           int32_t d_k, int32_t d_v, int32_t chunk_size,
                           kda_dtype dtype, const float *initial_state,
                           float *final_state, void *o, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * The two kernels of kda_fwd_chunked, in launch order.  Exposed so that a
 * caller can time or schedule them separately.
 */
typedef enum {
  KDA_STAGE_INTRA = 0, /* per chunk: cumulative log-decay, A, P, UT inverse,
                          WY factors W and U                             */
  KDA_STAGE_INTER = 1  /* state carried over chunks: o and final_state   */
} kda_fwd_stage;

/*
 * Enqueues one stage of kda_fwd_chunked with the same arguments and the
 * same validation.  kda_fwd_chunked == INTRA then INTER on one stream and
 * one workspace.  A stage reads what the earlier stages left in
 * the workspace, so it must follow them (stream order) with identical
 * arguments; re-running a stage on an unchanged workspace reproduces its
 * outputs (INTER is not idempotent when initial_state aliases final_state).
 */
kda_status kda_fwd_chunked_stage(kda_fwd_stage stage, const void *q, const void *k,
                                 const void *v, const float *log_alpha,
                                 const float *beta, const int32_t *cu_seqlens,
                                 int32_t num_seqs, int64_t total_tokens,
                                 int32_t num_heads, int32_t d_k, int32_t d_v,
                                 int32_t chunk_size, kda_dtype dtype,
                                 const float *initial_state, float *final_state,
                                 void *o, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * ---- Options of the _ex calls ---------------------------------------------
 * Input-side fusion: steps that the layers feeding the operator would
 * otherwise run as separate passes over q, k, the gate and beta, done by the
 * kernels as they read them (docsaid.org "Kimi Linear", section "Les autres
 * pieces": q and k are L2-normalised, beta is a sigmoid, the decay comes from
 * a gate function; fr.news.hada.io, section "Configuration du modele Kimi
 * Linear"; mkdocs.reaper.mx "Attention lineaire et recurrence", section "Le
 * piege numerique de la decroissance cumulee": Kimi Linear's
 * g = -exp(A) softplus(z), and the scaled sigmoid bounded below by g_min).
 * Output epilogue: the per-head RMSNorm and the data-dependent sigmoid
 * output gate that follow the operator (same docsaid.org section;
 * fr.news.hada.io, section "Configuration du modele Kimi Linear").
 * All of it is evaluated in fp32.
 */
typedef enum {
  KDA_GATE_LOG_ALPHA = 0, /* gate holds g = log(alpha) itself, fp32           */
  KDA_GATE_SOFTPLUS = 1,  /* gate holds z in dtype: g = -exp(A[h]) softplus(z),
                             softplus(z) = log(1 + exp(z))                     */
  KDA_GATE_SIGMOID = 2    /* gate holds z in dtype: g = gate_min sigmoid(z),
                             so g lies in (gate_min, 0)                        */
} kda_gate;

typedef struct {
  /* -- input-side fusion -- */
  kda_gate gate;
  const float *gate_A;  /* KDA_GATE_SOFTPLUS: [num_heads] fp32 device array  */
  float gate_min;       /* KDA_GATE_SIGMOID: finite and < 0 (-5 in Kimi K3)  */
  int32_t l2norm_qk;    /* nonzero: q <- q / sqrt(|q|^2 + 1e-6) per token and
                           head, and the same for k, before any other use   */
  int32_t beta_logits;  /* nonzero: beta holds logits b; beta = sigmoid(b)   */
  /* -- serving: state slots (a drop-in cache for continuous batching; the
     state per request has a fixed size, docsaid.org "Calculer le cache a la
     main").  NULL = state i belongs to sequence i.  Otherwise the state
     tensors (decode: state; prefill: initial_state and final_state) are
     pools of num_slots states [num_slots, H, d_k, d_v], and sequence i uses
     slot state_slots[i] (int32 device array, one entry per sequence).  A
     slot outside [0, num_slots) marks padding: decode writes o = 0 for it
     and leaves every state untouched; prefill starts it from a zero state
     and writes no final state.  Slots of different sequences must differ. */
  const int32_t *state_slots;
  int32_t num_slots;
  /* -- output epilogue: when out_norm_weight is set, every output row
     o[t, h, :] (d_v values) becomes
         o / sqrt(mean(o^2) + out_norm_eps) * out_norm_weight * sigmoid(z_o)
     with z_o = out_gate[t, h, :] (the sigmoid factor is 1 when out_gate is
     NULL).  Decode applies it to the fp32 output before rounding; prefill
     runs it as a pass over o after the inter-chunk kernel (its d_v columns
     are computed by different workgroups), within the inter stage.        */
  const float *out_norm_weight; /* [d_v] fp32, shared by the heads, or NULL */
  const void *out_gate;         /* [tokens or batch, H, d_v] in dtype, or NULL */
  float out_norm_eps;           /* > 0, finite                              */
  /* -- diagnostics (prefill).  flags: an int32 device word, 4-byte aligned,
     into which the prefill kernels OR the KDA_FLAG_* bits below; the caller
     zeroes it before the call and reads it after synchronising.  NULL = no
     diagnostics.  check_inputs != 0 (needs flags) first validates
     cu_seqlens on the device: cu[0] = 0, non-decreasing, cu[num_seqs] =
     total_tokens.  If that fails, KDA_FLAG_BAD_CU_SEQLENS is set and every
     prefill kernel of the call returns without reading the inputs or
     writing o, final_state or the workspace (contents that break the rules
     are otherwise undefined behaviour).  kda_decode_step_ex ignores both. */
  int32_t *flags;
  int32_t check_inputs;
} kda_options;

/* Bits of kda_options.flags. */
#define KDA_FLAG_DECAY_RANGE 1    /* some 16-token block's summed log-decay fell
                                     below -80 in a channel: outside the
                                     precondition of the chunk algorithm (see
                                     kda_fwd_chunked); that chunk's outputs may
                                     be inf/NaN.  Set by the intra-chunk kernel. */
#define KDA_FLAG_BAD_CU_SEQLENS 2 /* check_inputs: cu_seqlens failed
                                     validation; nothing was computed.        */

/*
 * kda_fwd_chunked with options (input-side fusion, state slots, output
 * epilogue) and a stage mask.
 *
 *   options  kda_options above; NULL (or all fields zero) is exactly
 *            kda_fwd_chunked.  out_gate is [total_tokens, H, d_v] in dtype,
 *            16-byte aligned.
 *   stages   bit 0 runs the intra-chunk kernel, bit 1 the inter-chunk
 *            kernel (3 = the whole call; see kda_fwd_chunked_stage for the
 *            ordering rules of single stages).  Other values are invalid.
 *   gate     [total_tokens, H, d_k]: fp32 g for KDA_GATE_LOG_ALPHA, else z
 *            in dtype (half the bytes of g for bf16).  16-byte aligned.
 *   beta     [total_tokens, H] fp32: beta, or its logits.
 * Every other argument is as for kda_fwd_chunked, and so is the decay
 * precondition, which now applies to the g the gate function produces.
 * KDA_GATE_SIGMOID with gate_min >= -5 meets it for any z and any chunk size
 * (16 x 5 = 80, the tile bound of the section cited above).
 */
kda_status kda_fwd_chunked_ex(const kda_options *options, uint32_t stages, const void *q,
                              const void *k, const void *v, const void *gate,
                              const float *beta, const int32_t *cu_seqlens,
                              int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                              int32_t d_k, int32_t d_v, int32_t chunk_size,
                              kda_dtype dtype, const float *initial_state,
                              float *final_state, void *o, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step for a batch of states, updated in place.
 * For each (b, h): S' = Diag(alpha) S; u = beta (v - S'^T k);
 * o = S'^T q + (k . q) u; S <- S' + k u^T -- the same update and read-out as
 * above for a single token (mkdocs.reaper.mx "Attention lineaire et
 * recurrence", section "Kimi Delta Attention = les trois remedes combines";
 * docsaid.org "Calculer le cache a la main": the state size does not depend
 * on the context length).  Each state is read once and written once.
 *
 *   q, k        [batch, H, d_k]  dtype
 *   v           [batch, H, d_v]  dtype
 *   log_alpha   [batch, H, d_k]  fp32 (finite, <= 0)
 *   beta        [batch, H]       fp32
 *   state       [batch, H, d_k, d_v] fp32, read and overwritten
 *   o           [batch, H, d_v]  dtype (output)
 *
 * q, k, v, o, log_alpha and state must be 16-byte aligned; beta 4-byte.
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           float *state, void *o, int32_t batch,
                           int32_t num_heads, int32_t d_k, int32_t d_v,
                           kda_dtype dtype, void *stream);

/*
 * kda_decode_step with options: `options` and `gate` as for
 * kda_fwd_chunked_ex (gate [batch, H, d_k], out_gate [batch, H, d_v];
 * NULL options = kda_decode_step).  With state_slots, `state` is the pool.
 */
kda_status kda_decode_step_ex(const kda_options *options, const void *q, const void *k,
                              const void *v, const void *gate, const float *beta,
                              float *state, void *o, int32_t batch, int32_t num_heads,
                              int32_t d_k, int32_t d_v, kda_dtype dtype, void *stream);

/*
 * ---- Prefill without any allocation -------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * kda_fwd_chunked_noalloc is kda_fwd_chunked (same arguments and kernels,
 * same results bit for bit) with the workspace taken from a device array
 * that the library holds on every GPU it runs on, until the process ends:
 * KDA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU.  It allocates nothing and calls
 * no allocating routine.  The first call on a device, with that device
 * current, looks up the array's device address (hipGetSymbolAddress); the
 * stream must belong to the current device.
 *
 *   Returns KDA_ERROR_SCRATCH_TOO_SMALL, with nothing enqueued, when
 *   kda_fwd_chunked_workspace_size() for the arguments exceeds
 *   KDA_NOALLOC_SCRATCH_BYTES (bf16, d = 128, C = 64 needs about 72.5 KiB
 *   per (chunk, head) tile: e.g. B=2 x T=2048 x H=8 takes 36.8 MiB), and
 *   KDA_ERROR_LAUNCH_FAILED if the array's address cannot be found.  Other
 *   errors are kda_fwd_chunked's.
 *   Calls on one GPU share its array: calls that overlap on one GPU (several
 *   streams or host threads at once) race and must be serialised by the
 *   caller.  Each call writes every workspace value it uses before using
 *   it, so nothing left by an earlier call affects the results.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

kda_status kda_fwd_chunked_noalloc(const void *q, const void *k, const void *v,
                                   const float *log_alpha, const float *beta,
                                   const int32_t *cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t num_heads, int32_t d_k,
                                   int32_t d_v, int32_t chunk_size, kda_dtype dtype,
                                   const float *initial_state, float *final_state, void *o,
                                   void *stream);

/*
 * ---- Backward (training) ----------------------------------------------------
 * Gradients of the chunked prefill (fr.news.hada.io Kimi Linear summary,
 * section "Algorithme parallele par chunks": the chunk form with the UT
 * transform is what training runs), for the loss
 *     L = sum(o * d_o) + sum(final_state * d_final_state).
 * The chunk factors and the chunk start states are recomputed from the
 * inputs; everything is evaluated in fp32.
 *
 *   q, k, v, log_alpha, beta, cu_seqlens, num_seqs, ..., initial_state:
 *                 as for kda_fwd_chunked (same values as the forward call).
 *   d_o           [total_tokens, H, d_v] dtype, the gradient of o.
 *   d_final_state [num_seqs, H, d_k, d_v] fp32, or NULL for zero.
 *   dq, dk        [total_tokens, H, d_k] dtype (outputs).
 *   dv            [total_tokens, H, d_v] dtype (output).
 *   dlog_alpha    [total_tokens, H, d_k] fp32 (output).
 *   dbeta         [total_tokens, H] fp32 (output).
 *   d_initial_state [num_seqs, H, d_k, d_v] fp32 (output), or NULL to skip.
 *   workspace     at least kda_bwd_chunked_workspace_size() bytes, 256-byte
 *                 aligned, clobbered (about 0.9 MiB per (chunk, head) tile
 *                 for d = 128, C = 64).
 * Alignment rules are those of kda_fwd_chunked (d_o, dq, dk, dv 16-byte;
 * dlog_alpha 16-byte; dbeta 4-byte).  The decay precondition is the
 * forward's.
 */
size_t kda_bwd_chunked_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                      int32_t num_heads, int32_t d_k, int32_t d_v,
                                      int32_t chunk_size, kda_dtype dtype);

kda_status kda_bwd_chunked(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const int32_t *cu_seqlens, int32_t num_seqs,
                           int64_t total_tokens, int32_t num_heads, int32_t d_k,
                           int32_t d_v, int32_t chunk_size, kda_dtype dtype,
                           const float *initial_state, const void *d_o,
                           const float *d_final_state, void *dq, void *dk, void *dv,
                           float *dlog_alpha, float *dbeta, float *d_initial_state,
                           void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
