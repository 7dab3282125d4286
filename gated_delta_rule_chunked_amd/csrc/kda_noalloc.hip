// kda_noalloc.hip -- kda_fwd_chunked for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): the prefill workspace is a file-scope device array,
// `scratch`, of KDA_NOALLOC_SCRATCH_BYTES on every GPU the library runs on,
// held until the process ends.  The kernels are those of kda_fwd_chunked;
// only the workspace pointer differs.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// its device address is looked up once per device with hipGetSymbolAddress
// (that device current) and only that address is ever passed to a kernel.
// Calls on one GPU share its array, so calls that overlap on one GPU race;
// the prefill writes every workspace value it uses within the call before
// using it, so the previous call's contents need no clearing.
#include <atomic>
#include <hip/hip_runtime.h>

#include "kda.h"

namespace {

static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_addr[kMaxDevices];  // zero-initialised: not looked up

// Device address of the current device's `scratch`, or nullptr if it cannot
// be found.  Concurrent first calls may both look it up, which is harmless.
void *device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();  // leave no sticky error for the caller's next call
    return nullptr;
  }
  scratch_addr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" kda_status kda_fwd_chunked_noalloc(
    const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
    const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
    int32_t d_k, int32_t d_v, int32_t chunk_size, kda_dtype dtype, const float *initial_state,
    float *final_state, void *o, void *stream) {
  const size_t need = kda_fwd_chunked_workspace_size(total_tokens, num_seqs, num_heads, d_k,
                                                     d_v, chunk_size, dtype);
  if (need == 0)  // invalid or unsupported sizes: kda_fwd_chunked names which
    return kda_fwd_chunked(q, k, v, log_alpha, beta, cu_seqlens, num_seqs, total_tokens,
                           num_heads, d_k, d_v, chunk_size, dtype, initial_state, final_state,
                           o, nullptr, 0, stream);
  if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERROR_SCRATCH_TOO_SMALL;
  void *ws = device_scratch();
  if (ws == nullptr) return KDA_ERROR_LAUNCH_FAILED;
  return kda_fwd_chunked(q, k, v, log_alpha, beta, cu_seqlens, num_seqs, total_tokens,
                         num_heads, d_k, d_v, chunk_size, dtype, initial_state, final_state, o,
                         ws, KDA_NOALLOC_SCRATCH_BYTES, stream);
}
