// lsh_device.h -- types and helpers shared by the gfx950 kernels of liblsh.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 64;   // d
constexpr int kChunk = 64;     // m
constexpr int kWave = 64;      // CDNA wavefront

// One dispatch may hold fewer than 2^32 work-items.  Kernels whose grid grows
// with the problem are launched in pieces of at most kMaxBlocks workgroups
// (2^30 work-items at 256 per workgroup), each told its first block.
constexpr int64_t kMaxBlocks = int64_t(1) << 22;

// Raw buffer descriptor word 3 for gfx9 (32-bit data format; no swizzle): a
// load at a byte offset past the descriptor's size returns zero.
constexpr int kBufferWord3 = 0x00020000;

// 16-byte global/LDS load and store through uint4.
__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void store16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8, u);
}

// bf16 halves of a packed dword -> fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 pair -> packed bf16 pair, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a = (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
  b = (b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u;
  return a | b;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// A pointer that is the same in every lane, marked as such (read from the
// first active lane), so that a buffer descriptor built from it stays in
// scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// The value of lane l ^ 32 (the other half of the wave), with one
// v_permlane32_swap (a VALU exchange of the two 32-lane halves) instead of an
// LDS permute.  Every lane of the wave must be active.
__device__ __forceinline__ uint32_t other_half(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  // r[0]: lanes 0-31 keep x, lanes 32-63 receive x of lanes 0-31;
  // r[1]: lanes 0-31 receive x of lanes 32-63, lanes 32-63 keep x
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float other_half(float x) {
  return __uint_as_float(other_half(__float_as_uint(x)));
}

// Maximum over the 64 lanes of a wave (every lane active), with no LDS
// address registers: DPP exchanges inside each row of 16 lanes (quad
// permutes for lane ^ 1 and lane ^ 2, then the half-row and row mirrors,
// which pair groups of 4 and of 8), ds_swizzle for lane ^ 16, and the
// 32-lane swap.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
  return fmaxf(v, other_half(v));
}

// Index read from caller memory, forced into [0, n) so that no input can make
// a kernel access memory outside its buffers.
__device__ __forceinline__ int clamp_index(int i, int n) { return min(max(i, 0), n - 1); }

// Workgroups are handed to the 8 XCDs of the chip round-robin (hardware block
// w runs on XCD w % 8).  This maps the hardware id to a logical block index so
// that each XCD works through one contiguous eighth of the logical range,
// keeping the data of neighbouring logical blocks in that XCD's own L2.
// It is a bijection on [0, n).
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_logical_block(int64_t w, int64_t n) {
  const int64_t x = w % kXcds, k = w / kXcds;
  const int64_t q = n / kXcds, rem = n % kXcds;
  return x * q + (x < rem ? x : rem) + k;
}

// Groups of `per` consecutive logical blocks ("units"): when the number of
// units is a multiple of 8, XCD x works through units x, x+8, x+16, ... in
// order, so at any moment the 8 XCDs hold 8 neighbouring units (for the
// attention: the 8 hash rounds of one head, whose x and v rows are then hot in
// the memory-side cache while each XCD's L2 keeps its own round's indices).
// Otherwise the plain order is used.  A bijection on [0, units * per).
__device__ __forceinline__ int64_t xcd_interleaved_block(int64_t w, int64_t units, int64_t per) {
  if (units % kXcds != 0) return w;
  const int64_t x = w % kXcds, k = w / kXcds;
  return (x + kXcds * (k / per)) * per + k % per;
}

// ---------------------------------------------------------------------------
// fp16 per-round outputs (bf16 inputs).  Every output row o is a weighted mean
// of v rows, so |o| <= max |v| of its (batch, head) up to the rounding of the
// mean.  The rows are stored as fp16 of o * 2^-k, where k = max(e - 15, -100)
// for the smallest e with max |v| < 2^e: each stored magnitude stays within
// rounding of 2^15, far below fp16's largest value 65504, and the scale is a
// power of two, so it adds no rounding of its own.
constexpr int kVParts = 256;   // partial maxima of |v| per (batch, head)

__device__ __forceinline__ int o_scale_exponent(float vmax) {
  const int biased = (int)(__float_as_uint(vmax) >> 23);   // vmax >= 0, finite
  const int e = biased == 0 ? -126 : biased - 126;
  return max(e - 15, -100);
}

// 2^k for -126 <= k <= 127.
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(127 + k) << 23); }

// The largest of one (batch, head)'s kVParts partial maxima (16-byte aligned),
// in every lane of the calling wave.
__device__ __forceinline__ float head_vmax(const float* part) {
  static_assert(kVParts == 4 * kWave, "one float4 per lane");
  const float4 p = *reinterpret_cast<const float4*>(part + 4 * (threadIdx.x & (kWave - 1)));
  float m = fmaxf(fmaxf(p.x, p.y), fmaxf(p.z, p.w));
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  return m;
}

}  // namespace lsh
