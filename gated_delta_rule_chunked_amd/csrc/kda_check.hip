// kda_check.hip -- on-device handling of cu_seqlens: its validation for the
// prefill, and the chunk table of packed sequences.
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

// The chunk table of packed sequences: chunk id -> (sequence, first token,
// rows), ids enumerating the chunks of sequence 0, then 1, ... (chunks never
// straddle sequences; a sequence's last chunk holds the tail).  One
// workgroup walks the sequences 1,024 at a time: chunk counts and a block
// scan give each sequence's first id; then every thread strides over the
// pass's chunk ids and finds its sequence by binary search in the scan, so a
// long sequence's entries are written by all threads at once.  Entries past
// the last chunk get rows = 0, so the tiles launched for the bound
// max_chunks that no chunk fills have nothing to do.  Lengths that break the
// rules (negative, or a range outside [0, total)) count as empty and ids at
// or past max_chunks are not written.
constexpr int kTabThreads = 1024;

__global__ __launch_bounds__(kTabThreads) void chunk_table_kernel(
    const int *__restrict__ cu, int N, int64_t total, int C, int64_t max_chunks,
    int4 *__restrict__ tab, int *__restrict__ seq_first, const OptArgs in) {
  if (inputs_rejected(in)) return;
  __shared__ long long s_scan[kTabThreads];  // inclusive chunk-count scan of the pass
  __shared__ int s_start[kTabThreads], s_len[kTabThreads];
  const int tid = threadIdx.x;
  long long base = 0;
  for (int s0 = 0; s0 < N; s0 += kTabThreads) {
    const int s = s0 + tid;
    const int ns = min(kTabThreads, N - s0);  // sequences in this pass
    int start = 0, len = 0;
    if (s < N) {
      start = cu[s];
      len = cu[s + 1] - start;
      if (start < 0 || len < 0 || (int64_t)start + len > total) len = 0;
    }
    const long long nc = (len + C - 1) / C;
    s_scan[tid] = nc;
    s_start[tid] = start;
    s_len[tid] = len;
    __syncthreads();
    for (int off = 1; off < kTabThreads; off <<= 1) {
      const long long add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    if (s < N) {
      const long long first = base + s_scan[tid] - nc;
      seq_first[s] = (int)(first < max_chunks ? first : max_chunks);
    }
    const long long pass_chunks = s_scan[kTabThreads - 1];
    for (long long e = tid; e < pass_chunks && base + e < max_chunks; e += kTabThreads) {
      // the sequence slot holding chunk e of the pass: the first slot whose
      // inclusive count exceeds e (empty sequences never qualify)
      int lo = 0, hi = ns - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_scan[mid] > e) hi = mid;
        else lo = mid + 1;
      }
      const int i = (int)(e - (lo > 0 ? s_scan[lo - 1] : 0));  // chunk index in its sequence
      tab[base + e] = make_int4(s0 + lo, s_start[lo] + i * C, min(C, s_len[lo] - i * C), 0);
    }
    base += pass_chunks;
    __syncthreads();
  }
  for (long long c = base + tid; c < max_chunks; c += kTabThreads) tab[c] = make_int4(N, 0, 0, 0);
}

hipError_t launch_chunk_table(const int *cu, int N, int64_t total, int C, int64_t max_chunks,
                              int4 *tab, int *seq_first, const OptArgs &in, hipStream_t stream) {
  if (max_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kTabThreads), 0, stream, cu, N, total, C,
                     max_chunks, tab, seq_first, in);
  return hipGetLastError();
}

hipError_t launch_check_cu(const int *cu, int N, int64_t total, int *flags,
                           hipStream_t stream) {
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, stream, cu, N, total, flags);
  return hipGetLastError();
}

}  // namespace kda
