// kda_epilogue.hip -- the output epilogue of the prefill: per-head RMSNorm
// and the data-dependent sigmoid output gate, in place on o,
//   o[r, :] <- o[r, :] / sqrt(mean(o[r, :]^2) + eps) * w * sigmoid(z[r, :])
// for every (token, head) row r (docsaid.org "Kimi Linear", section "Les
// autres pieces": RMSNorm per head, then a sigmoid gate that depends on the
// input; fr.news.hada.io, section "Configuration du modele Kimi Linear").
//
// The inter-chunk kernel computes the d_v columns of a row in different
// workgroups (the state is sliced by columns to spread the serial chain over
// the GPU), so the row statistics need this pass.  It reads o and z once and
// writes o once: bound by HBM bandwidth.  Lanes hold 8 consecutive values
// (one 16-byte access for bf16); the d/8 lanes of a row sum their squares
// with lane exchanges.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <typename T, int D>
__global__ __launch_bounds__(256) void out_epilogue_kernel(T *__restrict__ o,
                                                           const T *__restrict__ z,
                                                           const float *__restrict__ w,
                                                           float eps, int64_t rows,
                                                           const OptArgs in) {
  if (inputs_rejected(in)) return;
  constexpr int L = D / 8;        // lanes per row
  constexpr int RPB = 256 / L;    // rows per block
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / L;
  const int c0 = (threadIdx.x % L) * 8;
  const bool live = r < rows;     // every lane takes part in the row sums
  const int64_t at = (live ? r : 0) * D + c0;
  const f32x4 x0 = to_f32x4(load4<T>(o + at)), x1 = to_f32x4(load4<T>(o + at + 4));
  float ss = x0[0] * x0[0] + x0[1] * x0[1] + x0[2] * x0[2] + x0[3] * x0[3] +
             x1[0] * x1[0] + x1[1] * x1[1] + x1[2] * x1[2] + x1[3] * x1[3];
  ss = group_sum<L>(ss);
  const float s = rsqrtf(ss * (1.f / D) + eps);
  f32x4 y0 = x0 * s * *reinterpret_cast<const f32x4 *>(w + c0);
  f32x4 y1 = x1 * s * *reinterpret_cast<const f32x4 *>(w + c0 + 4);
  if (z) {
    const f32x4 z0 = to_f32x4(load4<T>(z + at)), z1 = to_f32x4(load4<T>(z + at + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y0[e] *= sigmoid(z0[e]);
      y1[e] *= sigmoid(z1[e]);
    }
  }
  if (live) store8_f32<T>(o + at, y0, y1);
}

template <typename T, int D>
static hipError_t launch_epi(void *o, const OptArgs &in, int64_t rows, hipStream_t s) {
  constexpr int RPB = 256 / (D / 8);
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  hipLaunchKernelGGL((out_epilogue_kernel<T, D>), grid, dim3(256), 0, s,
                     reinterpret_cast<T *>(o), reinterpret_cast<const T *>(in.out_gate),
                     in.norm_w, in.norm_eps, rows, in);
  return hipGetLastError();
}

hipError_t launch_out_epilogue(void *o, const OptArgs &in, int64_t rows, int d, kda_dtype dt,
                               hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (dt == KDA_DTYPE_BF16) {
    switch (d) {
      case 32: return launch_epi<bf16, 32>(o, in, rows, stream);
      case 64: return launch_epi<bf16, 64>(o, in, rows, stream);
      case 128: return launch_epi<bf16, 128>(o, in, rows, stream);
    }
  } else {
    switch (d) {
      case 32: return launch_epi<float, 32>(o, in, rows, stream);
      case 64: return launch_epi<float, 64>(o, in, rows, stream);
      case 128: return launch_epi<float, 128>(o, in, rows, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
