// kda_common.hpp -- device-side building blocks shared by the KDA kernels:
// element types, 16x16 MFMA tiles for gfx950, fragment loads and
// conversions.
//
// Matrix-core tile convention (verified on gfx950 for both instructions):
// a 16 x 16 output tile D = A (16 x K) * B (K x 16) is accumulated over
// K-steps of 32.  In each K-step, lane l (0..63) supplies eight A values
// A[l % 16][8 * (l / 16) + i] and eight B values B[8 * (l / 16) + i][l % 16],
// i = 0..7, and holds the four outputs D[4 * (l / 16) + i][l % 16], i = 0..3.
//   bf16: one v_mfma_f32_16x16x32_bf16 per K-step.
//   fp32: eight v_mfma_f32_16x16x4_f32, instruction i taking element i; each
//         covers k = 8 * (l / 16) + i over the four lane groups, so the eight
//         together cover the same 32 values of k.
// Both A and B fragments are therefore eight CONTIGUOUS elements of a row of
// a row-major buffer (A stored [m][k], B stored transposed as [n][k]).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x4 mma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_k32(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

// fp32 16x16x16 product step (K = 16): lane l supplies A[l%16][4*(l/16)+i]
// and B[4*(l/16)+i][l%16] for i = 0..3 through four 16x16x4 instructions.
__device__ __forceinline__ f32x4 mma_f32_k16(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- conversions -------------------------------------------------------
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ---- 8-element contiguous loads/stores (16 B for bf16, 32 B for fp32) --
template <typename T>
__device__ __forceinline__ typename Frag<T>::type load8(const T *p);

template <>
__device__ __forceinline__ bf16x8 load8<bf16>(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
template <>
__device__ __forceinline__ f32x8 load8<float>(const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename T>
__device__ __forceinline__ void store8(T *p, const float (&x)[8]);
template <>
__device__ __forceinline__ void store8<bf16>(bf16 *p, const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)x[i];
  *reinterpret_cast<bf16x8 *>(p) = r;
}
template <>
__device__ __forceinline__ void store8<float>(float *p, const float (&x)[8]) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4 *>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// 8 fp32 values converted to a fragment of T.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type frag_from_f32(const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  typename Frag<T>::type r;
  r[0] = from_f32<T>(a[0]); r[1] = from_f32<T>(a[1]);
  r[2] = from_f32<T>(a[2]); r[3] = from_f32<T>(a[3]);
  r[4] = from_f32<T>(b[0]); r[5] = from_f32<T>(b[1]);
  r[6] = from_f32<T>(b[2]); r[7] = from_f32<T>(b[3]);
  return r;
}

// 4 consecutive elements kept in the element type (convert at use, so that a
// prefetching load does not force an early wait).
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };
template <typename T>
__device__ __forceinline__ typename Vec4<T>::type load4(const T *p) {
  return *reinterpret_cast<const typename Vec4<T>::type *>(p);
}
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 to_f32x4(f32x4 v) { return v; }

// 4 consecutive elements (one D-layout column strip) as fp32 / from fp32.
template <typename T>
__device__ __forceinline__ f32x4 load4_f32(const T *p);
template <>
__device__ __forceinline__ f32x4 load4_f32<bf16>(const bf16 *p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <>
__device__ __forceinline__ f32x4 load4_f32<float>(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}
template <typename T>
__device__ __forceinline__ void store4_f32(T *p, f32x4 x);
template <>
__device__ __forceinline__ void store4_f32<bf16>(bf16 *p, f32x4 x) {
  *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}
template <>
__device__ __forceinline__ void store4_f32<float>(float *p, f32x4 x) {
  *reinterpret_cast<f32x4 *>(p) = x;
}

// ---- contraction order of the register-resident state chain -----------
// A 16 x 16 output tile leaves lane l holding rows 4 * (l / 16) + i,
// i = 0..3, while a K-step wants lane l to supply k = 8 * (l / 16) + i,
// i = 0..7.  Because a contraction may visit k in any order (as long as
// both operands agree), two stacked output tiles (rows 0..15 and 16..31 of
// a 32-group) can serve directly as one K-step operand if, within every
// group of 32, storage position p = 8 * g + j holds index
// j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4).  Matrices that meet such
// register-held operands in a product are stored with their contraction
// index in this order.
__host__ __device__ constexpr int kperm_pos(int idx) {  // index -> position
  return (idx & ~31) + ((idx & 31) < 16 ? 8 * ((idx & 15) >> 2) + (idx & 3)
                                         : 8 * ((idx & 15) >> 2) + 4 + (idx & 3));
}
__host__ __device__ constexpr int kperm_idx(int pos) {  // position -> index
  return (pos & ~31) + (((pos & 7) < 4) ? 4 * ((pos & 31) >> 3) + (pos & 3)
                                        : 16 + 4 * ((pos & 31) >> 3) + (pos & 3));
}
// the two maps are inverse permutations of every group of 32
constexpr bool kperm_is_permutation() {
  for (int i = 0; i < 64; ++i)
    if (kperm_idx(kperm_pos(i)) != i || kperm_pos(kperm_idx(i)) != i) return false;
  return true;
}
static_assert(kperm_is_permutation(), "kperm order");

// Two output-tile row quads (rows 4g..4g+3 of tiles 2s and 2s+1) packed as
// one K-step operand fragment in the order above.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type pack_quads(f32x4 a, f32x4 b) {
  typename Frag<T>::type r;
  r[0] = from_f32<T>(a[0]); r[1] = from_f32<T>(a[1]);
  r[2] = from_f32<T>(a[2]); r[3] = from_f32<T>(a[3]);
  r[4] = from_f32<T>(b[0]); r[5] = from_f32<T>(b[1]);
  r[6] = from_f32<T>(b[2]); r[7] = from_f32<T>(b[3]);
  return r;
}

// 8 consecutive elements from two fp32 quads (16 bytes for bf16).
template <typename T>
__device__ __forceinline__ void store8_f32(T *p, f32x4 a, f32x4 b) {
  *reinterpret_cast<typename Frag<T>::type *>(p) = pack_quads<T>(a, b);
}

// ---- fragment-major workspace storage -------------------------------------
// An operand that one kernel writes and another feeds to the matrix cores is
// stored in the order its fragments are loaded, so that each wavefront load
// is one contiguous run (1 KiB for bf16) instead of 16 half-used cache lines.
// K-step operand (rows, contraction positions pos in [0, K), K % 32 == 0):
// the 8-element fragment of lane l for row block rb and K-step ks is run
// (rb * K/32 + ks) * 64 + l, lane l covering row 16 rb + l % 16 and
// positions 32 ks + 8 (l / 16) + e.
__host__ __device__ constexpr int frag_off(int row, int pos, int K) {
  return ((row >> 4) * (K >> 5) + (pos >> 5)) * 512 +
         ((((pos & 31) >> 3) << 4) + (row & 15)) * 8 + (pos & 7);
}
// Output-tile operand (tokens t in [0, C), columns c): the 4 values lane l
// holds of 16x16 tile (column block c / 16, token block t / 16) are run
// (c/16 * C/16 + t/16) * 64 + l, lane l covering column 16 (c/16) + l % 16
// and tokens 16 (t/16) + 4 (l / 16) + i.
__host__ __device__ constexpr int tile_off(int t, int c, int C) {
  return ((c >> 4) * (C >> 4) + (t >> 4)) * 256 +
         ((((t & 15) >> 2) << 4) + (c & 15)) * 4 + (t & 3);
}

// Two 4-element vectors joined into one 8-element fragment.
__device__ __forceinline__ bf16x8 join4(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 join4(f32x4 a, f32x4 b) {
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <typename T>
__device__ __forceinline__ typename Vec4<T>::type vec4_from_f32(f32x4 x) {
  typename Vec4<T>::type r;
  r[0] = from_f32<T>(x[0]); r[1] = from_f32<T>(x[1]);
  r[2] = from_f32<T>(x[2]); r[3] = from_f32<T>(x[3]);
  return r;
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also
// carries a workgroup-scope release fence, which waits for every outstanding
// global load as well and so would drain loads issued ahead of their use.
// Here each wave's LDS writes complete (lgkmcnt 0) before it joins the
// barrier; the memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Lane index helpers for the tile convention above.
// ---- input-side fusion (kda_options in kda.h), fp32 ------------------------
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

// Kimi Linear's gate g = -exp(A) softplus(z), softplus(z) = log(1 + e^z)
// written as max(z, 0) + log(1 + e^-|z|) so that no exponential overflows.
__device__ __forceinline__ float gate_softplus(float z, float eA) {
  return -eA * (fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z))));
}
__device__ __forceinline__ f32x4 gate_softplus(f32x4 z, float eA) {
  return f32x4{gate_softplus(z[0], eA), gate_softplus(z[1], eA), gate_softplus(z[2], eA),
               gate_softplus(z[3], eA)};
}

// The bounded gate g = g_min sigmoid(z): in (g_min, 0) mathematically; in
// fp32 sigmoid rounds to 1 for z above about 17, so g can equal g_min.
__device__ __forceinline__ float gate_sigmoid(float z, float gmin) { return gmin * sigmoid(z); }
__device__ __forceinline__ f32x4 gate_sigmoid(f32x4 z, float gmin) {
  return f32x4{gmin * sigmoid(z[0]), gmin * sigmoid(z[1]), gmin * sigmoid(z[2]),
               gmin * sigmoid(z[3])};
}

// x + (x of the lane that the DPP control selects), within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W consecutive lanes (W = 4, 8, 16, 32 or 64),
// every lane of a group receiving the group's sum.  Pairwise exchanges:
// quad permutes [1,0,3,2] and [2,3,0,1], then the half-row mirror (lane i
// with 7 - i) and the row mirror (i with 15 - i), each pairing two groups
// whose sums are already complete; beyond 16 lanes a cross-lane shuffle.
template <int W>
__device__ __forceinline__ float group_sum(float s) {
  static_assert(W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
  s = dpp_add<0xB1>(s);   // quad_perm [1,0,3,2]
  s = dpp_add<0x4E>(s);   // quad_perm [2,3,0,1]
  if constexpr (W >= 8) s = dpp_add<0x141>(s);  // row_half_mirror
  if constexpr (W >= 16) s = dpp_add<0x140>(s);  // row_mirror
  if constexpr (W >= 32) s += __shfl_xor(s, 16);
  if constexpr (W >= 64) s += __shfl_xor(s, 32);
  return s;
}

// 1 / sqrt(|x|^2 + 1e-6) for a vector whose d channels sit 4 per lane in W
// consecutive lanes (W = d / 4, lane groups aligned to W).
template <int W>
__device__ __forceinline__ float l2_inv_norm(f32x4 x) {
  return rsqrtf(group_sum<W>(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]) + 1e-6f);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---- chunk location -------------------------------------------------------
// Sequence, first token and rows of chunk id c (rows = 0 past the last
// chunk).  Packed sequences read the chunk table built once per call
// (chunk_table_kernel); equal-length sequences compute it.  c is uniform
// over the workgroup, so the results are moved to scalar registers.
struct ChunkLoc {
  int seq, t0, n;
};
__device__ __forceinline__ ChunkLoc chunk_loc(int c, const int4 *tab, int N, int seq_len,
                                              int C) {
  ChunkLoc l;
  if (tab != nullptr) {
    const int4 e = tab[c];
    l.seq = e.x;
    l.t0 = e.y;
    l.n = e.z;
  } else {
    const int per = max((seq_len + C - 1) / C, 1);
    l.seq = c / per;
    const int i = c - l.seq * per;
    l.t0 = l.seq * seq_len + i * C;
    l.n = l.seq < N ? min(C, seq_len - i * C) : 0;
  }
  l.seq = __builtin_amdgcn_readfirstlane(l.seq);
  l.t0 = __builtin_amdgcn_readfirstlane(l.t0);
  l.n = __builtin_amdgcn_readfirstlane(l.n);
  return l;
}

}  // namespace kda
