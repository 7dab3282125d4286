// kda_cumsum.hip -- per-chunk cumulative log-decay and the chunk table.
//
// Inside a chunk the algorithm needs the cumulative decay of every key
// channel, gamma_r = alpha_1 ... alpha_r (mkdocs.reaper.mx "Attention
// lineaire et recurrence", section "Le piege numerique de la decroissance
// cumulee").  It is kept as its logarithm G_r = g_1 + ... + g_r, which is a
// plain prefix sum that restarts at every chunk start and every sequence
// start.  The same launch records, for every chunk id, which sequence it
// belongs to, its first token and its row count, so that the intra- and
// inter-chunk kernels need no host synchronisation for varlen batches.
//
// Grid: (chunk ids, heads); 256 threads.  Each thread owns one float4 column
// of the channel dimension and a contiguous run of rows: it sums its rows,
// the per-run totals are scanned through LDS, and every row is written once.
// Loads and stores are 16-byte and coalesced along the channel dimension.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

// Locates chunk id `c` among the sequences.  Writes (seq, first token, rows)
// into s_loc (rows = 0 if c is past the last chunk) and, for the block that
// owns the first chunk of a sequence and head 0, records seq_first.
__device__ void locate_chunk(int c, int h, const int *cu, int N, int seq_len,
                             int C, int *s_loc, int *s_scan, int *seq_first) {
  const int tid = threadIdx.x;
  if (cu == nullptr) {
    if (tid == 0) {
      const int per = (seq_len + C - 1) / C;
      const int s = c / per, i = c % per;
      const int rows = min(C, seq_len - i * C);
      s_loc[0] = s;
      s_loc[1] = s * seq_len + i * C;
      s_loc[2] = (s < N) ? rows : 0;
      if (h == 0 && i == 0 && s < N) seq_first[s] = c;
    }
    __syncthreads();
    return;
  }
  if (tid == 0) { s_loc[0] = 0; s_loc[1] = 0; s_loc[2] = 0; s_loc[3] = 0; }
  int base = 0;
  for (int s0 = 0; s0 < N; s0 += blockDim.x) {
    const int s = s0 + tid;
    int len = 0, start = 0;
    if (s < N) {
      start = cu[s];
      len = cu[s + 1] - start;
    }
    const int nc = (len + C - 1) / C;
    __syncthreads();
    s_scan[tid] = nc;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
      const int add = (tid >= off) ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    const int incl = base + s_scan[tid];
    const int excl = incl - nc;
    if (s < N && nc > 0) {
      if (c >= excl && c < incl) {
        const int i = c - excl;
        s_loc[0] = s;
        s_loc[1] = start + i * C;
        s_loc[2] = min(C, len - i * C);
        s_loc[3] = 1;
      }
      if (h == 0 && c == excl) seq_first[s] = c;
    }
    base += s_scan[blockDim.x - 1];
    __syncthreads();
    if (s_loc[3]) break;
  }
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(
    const float *__restrict__ g, const int *__restrict__ cu, int N, int H,
    int seq_len, int C, float *__restrict__ gc, int4 *__restrict__ chunk_info,
    int *__restrict__ seq_first) {
  constexpr int NCOL = D / 4;         // float4 columns per row
  constexpr int NRG = 256 / NCOL;     // row runs
  __shared__ int s_loc[4];
  __shared__ int s_scan[256];
  __shared__ f32x4 s_tot[NRG][NCOL];

  const int c = blockIdx.x, h = blockIdx.y;
  locate_chunk(c, h, cu, N, seq_len, C, s_loc, s_scan, seq_first);
  const int seq = s_loc[0], t0 = s_loc[1], rows = s_loc[2];
  if (h == 0 && threadIdx.x == 0) chunk_info[c] = int4{seq, t0, rows, 0};
  if (rows == 0) return;

  const int tid = threadIdx.x;
  const int col = tid % NCOL, rg = tid / NCOL;
  const int rpg = (C + NRG - 1) / NRG;  // rows per run
  const int r0 = rg * rpg;
  const int64_t row_stride = (int64_t)H * D;
  const float *src = g + ((int64_t)t0 * H + h) * D + 4 * col;
  float *dst = gc + ((int64_t)t0 * H + h) * D + 4 * col;

  f32x4 acc = zero4();
  for (int j = 0; j < rpg; ++j) {
    const int r = r0 + j;
    if (r < rows) acc += *reinterpret_cast<const f32x4 *>(src + r * row_stride);
  }
  s_tot[rg][col] = acc;
  __syncthreads();
  f32x4 run = zero4();
  for (int i = 0; i < rg; ++i) run += s_tot[i][col];
  for (int j = 0; j < rpg; ++j) {
    const int r = r0 + j;
    if (r < rows) {
      run += *reinterpret_cast<const f32x4 *>(src + r * row_stride);
      *reinterpret_cast<f32x4 *>(dst + r * row_stride) = run;
    }
  }
}

hipError_t launch_chunk_cumsum(const FwdArgs &a) {
  if (a.grid_chunks == 0) return hipSuccess;
  const dim3 grid((unsigned)a.grid_chunks, (unsigned)a.num_heads);
  float *gc = reinterpret_cast<float *>(a.ws + a.lay.gc);
  int4 *info = reinterpret_cast<int4 *>(a.ws + a.lay.chunk_info);
  int *first = reinterpret_cast<int *>(a.ws + a.lay.seq_first);
  switch (a.d) {
    case 32:
      hipLaunchKernelGGL(chunk_cumsum_kernel<32>, grid, dim3(256), 0, a.stream,
                         a.g, a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len,
                         a.chunk, gc, info, first);
      break;
    case 64:
      hipLaunchKernelGGL(chunk_cumsum_kernel<64>, grid, dim3(256), 0, a.stream,
                         a.g, a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len,
                         a.chunk, gc, info, first);
      break;
    case 128:
      hipLaunchKernelGGL(chunk_cumsum_kernel<128>, grid, dim3(256), 0, a.stream,
                         a.g, a.cu_seqlens, a.num_seqs, a.num_heads, a.seq_len,
                         a.chunk, gc, info, first);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kda
