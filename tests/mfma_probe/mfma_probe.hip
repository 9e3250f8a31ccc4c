// mfma_probe.hip -- test-only gfx950 kernel that exposes the raw fp32 results
// of the bf16 matrix-core contraction the bucket hash relies on.
//
// The bucket of a token is the first maximum of [x R ; -x R] with x R defined
// as an exact (fp64) sum (Reformer study note, section "LSH Attention": the
// hash into B buckets).  The library scores x R on v_mfma_f32_32x32x16_bf16
// and accepts a row only when the gap between its two best scores exceeds
// twice an assumed bound on the accumulation error.  This probe computes the
// same 64-term dot products with the same instruction, the same operand
// layout and the same accumulation sequence (four K = 16 steps from a zero
// accumulator), and writes every score, so that a test can measure the real
// error against the exact sums.  A second kernel computes the same dot
// products the way the hash recomputes the scores of a row's winning
// directions (two lanes per product, each a chain of 16 v_dot2_f32_bf16 over
// its 32 k-values, then the sum of the two halves).  It is not part of the
// library.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One wave per (32 tokens, 32 directions) tile; four waves per workgroup take
// four consecutive direction tiles.  x [n_tok][64] and r [n_dir][64] are bf16
// rows; out [n_tok][n_dir] fp32.  n_tok % 32 == 0 and n_dir % 128 == 0 (the
// host entry point checks both).
__global__ __launch_bounds__(256) void probe_scores_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ r,
                                                           float* __restrict__ out, int n_dir) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int jt = blockIdx.x * 4 + wave;   // direction tile
  const int tt = blockIdx.y;              // token tile
  bf16x8 a[4], b[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    // A: lane holds R[k = 8 (lane / 32) + 16 ks + 0..7][direction 32 jt + lane % 32]
    a[ks] = *reinterpret_cast<const bf16x8*>(r + (size_t)(32 * jt + (lane & 31)) * 64 +
                                             8 * (lane >> 5) + 16 * ks);
    // B: lane holds x[token 32 tt + lane % 32][k = 8 (lane / 32) + 16 ks + 0..7]
    b[ks] = *reinterpret_cast<const bf16x8*>(x + (size_t)(32 * tt + (lane & 31)) * 64 +
                                             8 * (lane >> 5) + 16 * ks);
  }
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], b[ks], acc, 0, 0, 0);
  // register i of lane l: direction 32 jt + 8 (i / 4) + 4 (l / 32) + i % 4, token l % 32
  const int tok = 32 * tt + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int dir = 32 * jt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    out[(size_t)tok * n_dir + dir] = acc[i];
  }
}

// Dot product p = (token p / n_dir, direction p % n_dir) by lanes p % 32 and
// p % 32 + 32 of a wave: lane half h takes k = 8 h + 16 ks + 0..7, ks = 0..3,
// in that order, two products per step; out[p] = half 0 + half 1.  The grid
// covers n_tok * n_dir products exactly (a multiple of 128).
__global__ __launch_bounds__(256) void probe_dots_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ r,
                                                         float* __restrict__ out, int n_dir) {
  const int lane = threadIdx.x & 63;
  const int64_t p = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 32 + (lane & 31);
  const int64_t tok = p / n_dir;
  const int dir = (int)(p % n_dir);
  const int h = lane >> 5;
  float part = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + tok * 64 + 8 * h + 16 * ks);
    const uint4 rv = *reinterpret_cast<const uint4*>(r + (int64_t)dir * 64 + 8 * h + 16 * ks);
    part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.x), __builtin_bit_cast(bf16x2, rv.x), part, false);
    part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.y), __builtin_bit_cast(bf16x2, rv.y), part, false);
    part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.z), __builtin_bit_cast(bf16x2, rv.z), part, false);
    part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.w), __builtin_bit_cast(bf16x2, rv.w), part, false);
  }
  const float v = part + __shfl_xor(part, 32);
  if (lane < 32) out[p] = v;
}

// Returns 0 on success, 1 on a shape the kernel does not take, 2 on a HIP
// error.  Pointers are device memory; the launch is on `stream`.
extern "C" int mfma_probe_scores(const void* x, const void* r, float* out, int n_tok, int n_dir,
                                 void* stream) {
  if (!x || !r || !out || n_tok <= 0 || n_dir <= 0 || n_tok % 32 || n_dir % 128 ||
      n_tok / 32 > 65535)
    return 1;
  hipLaunchKernelGGL(probe_scores_kernel, dim3(n_dir / 128, n_tok / 32), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(r), out, n_dir);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The same products through probe_dots_kernel; same shape rules and returns.
extern "C" int mfma_probe_dots(const void* x, const void* r, float* out, int n_tok, int n_dir,
                               void* stream) {
  if (!x || !r || !out || n_tok <= 0 || n_dir <= 0 || n_tok % 32 || n_dir % 128 ||
      (int64_t)n_tok * n_dir / 128 > 0x7fffffff)
    return 1;
  const int64_t blocks = (int64_t)n_tok * n_dir / 128;
  hipLaunchKernelGGL(probe_dots_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(r), out, n_dir);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
