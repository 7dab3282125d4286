// kda_check.hip -- on-device validation of cu_seqlens for the prefill.
//
// The sequence offsets are device data, so the host cannot check them
// without a synchronisation.  With kda_options.check_inputs this kernel runs
// first on the call's stream: one workgroup reads cu[0 .. N] once and ORs
// KDA_FLAG_BAD_CU_SEQLENS into the caller's flag word when cu[0] != 0, an
// offset decreases, or cu[N] != total_tokens.  Every prefill kernel of the
// call then returns at its start (inputs_rejected), so offsets that would
// index past the tensors are never used.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

__global__ __launch_bounds__(256) void check_cu_kernel(const int *__restrict__ cu, int N,
                                                       int64_t total, int *__restrict__ flags) {
  bool bad = false;
  for (int s = threadIdx.x; s < N; s += blockDim.x) bad |= cu[s + 1] < cu[s];
  if (threadIdx.x == 0) bad |= cu[0] != 0 || (int64_t)cu[N] != total;
  if (__syncthreads_or(bad) && threadIdx.x == 0) atomicOr(flags, KDA_FLAG_BAD_CU_SEQLENS);
}

hipError_t launch_check_cu(const int *cu, int N, int64_t total, int *flags,
                           hipStream_t stream) {
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, stream, cu, N, total, flags);
  return hipGetLastError();
}

}  // namespace kda
