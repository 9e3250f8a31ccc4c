// combine.hip -- unsort and combine the hash rounds (Reformer study note,
// section "Multiple Hash Rounds": the neighbourhood of a token is the union of
// its per-round neighbourhoods).  Taken as a multiset, the softmax over the
// union is the rounds' softmaxes merged with weights exp(lse_r - M) / sum.
//
// 16 lanes per token (4 features of the 64-wide row each); a 256-thread
// workgroup covers 16 consecutive tokens of one (batch, head), so y is written
// with full 256-byte rows while the per-round rows are gathered through
// inv_perm.  The per-round rows are fp32, or (compact format, bf16 inputs)
// fp16 of o * 2^-k with one k per (batch, head), read from the header of the
// per-round buffer; 2^k is applied once, with the normalisation.
#include <math.h>

#include <algorithm>

#include "lsh_device.h"
#include "lsh_launch.h"

namespace lsh {

template <typename T>
__device__ __forceinline__ float4 load_v4(const T* row, int c4);
template <>
__device__ __forceinline__ float4 load_v4<uint16_t>(const uint16_t* row, int c4) {
  const uint2 u = *reinterpret_cast<const uint2*>(row + c4);
  return make_float4(bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y));
}
template <>
__device__ __forceinline__ float4 load_v4<float>(const float* row, int c4) {
  return *reinterpret_cast<const float4*>(row + c4);
}

// Every per-round row is read once and every y row written once, so neither
// gains from staying in a cache: both go through non-temporal accesses
// (measured: the combine at 8 x 65,536 tokens, 8 rounds, 148 -> 137 us).
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store_y_nt(float* p, float4 v) {
  const f32x4v w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4v*>(p));
}
// bf16 outputs (the reversible layer's attention output, which its output
// map reads as bf16 anyway): rounded to nearest even, like that map's own
// rounding of fp32 inputs, so the layer's results do not change
__device__ __forceinline__ void store_y_nt(uint16_t* p, float4 v) {
  const bf16x2 lo = {(__bf16)v.x, (__bf16)v.y}, hi = {(__bf16)v.z, (__bf16)v.w};
  const u32x2v w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2v*>(p));
}

// Per-round rows: fp32, or fp16 in the compact format (O16).
template <bool O16>
struct ORows;
template <>
struct ORows<false> {
  typedef float elem;
  __device__ static float4 load4(const float* row, int c4) {
    const f32x4v w = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(row + c4));
    return make_float4(w.x, w.y, w.z, w.w);
  }
};
template <>
struct ORows<true> {
  typedef uint16_t elem;
  __device__ static float4 load4(const uint16_t* row, int c4) {
    const u32x2v w = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(row + c4));
    const uint2 u = make_uint2(w.x, w.y);
    const half2v lo = __builtin_bit_cast(half2v, u.x), hi = __builtin_bit_cast(half2v, u.y);
    return make_float4((float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y);
  }
};

// 2^k of (batch, head) bh (1 for fp32 rows).
template <bool O16>
__device__ __forceinline__ float o_unscale(const int32_t* hexp, int64_t bh) {
  if (!O16) return 1.0f;
  return pow2f(hexp[bh]);
}

// RMAX >= rounds: every round's slot, lse and output row are requested before
// any is used, so a token's R row gathers are in flight together.
template <typename T, bool O16, int RMAX, typename Y>
__global__ __launch_bounds__(256) void combine_kernel(
    const typename ORows<O16>::elem* __restrict__ o_rounds, const int32_t* __restrict__ hexp,
    const float* __restrict__ lse, const int32_t* __restrict__ inv_perm, const T* __restrict__ v,
    Y* __restrict__ y, int rounds, int L, int64_t total, int64_t blk0) {
  // Last tokens first: the per-round rows written last by the attention step
  // are the likeliest to still sit in the memory-side cache.
  const int64_t tok0 = (blk0 + gridDim.x - 1 - blockIdx.x) * 16;   // < total
  // the workgroup's 16 tokens lie in one (batch, head) (L is a multiple of 64)
  const float unscale = o_unscale<O16>(hexp, tok0 / L);
  const int64_t tok = tok0 + (threadIdx.x >> 4);
  if (tok >= total) return;
  const int c4 = (threadIdx.x & 15) * 4;
  const int64_t bh = tok / L;
  const int i = (int)(tok % L);
  const int64_t seg0 = bh * rounds;

  // The loads are unconditional so that they are all in flight at once:
  // slots past the last round repeat the last round's addresses (ignored).
  int64_t row[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int64_t seg = seg0 + (r < rounds ? r : rounds - 1);
    row[r] = seg * L + clamp_index(inv_perm[seg * L + i], L);
  }
  float l[RMAX];
  float4 o[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    l[r] = lse[row[r]];
    o[r] = ORows<O16>::load4(o_rounds + row[r] * kHeadDim, c4);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    if (r < rounds) mx = fmaxf(mx, l[r]);
  float4 out;
  if (mx == -INFINITY) {
    out = load_v4<T>(v + tok * kHeadDim, c4);
  } else {
    float ws = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r < rounds) {
        const float w = expf(l[r] - mx);
        ws += w;
        acc.x = fmaf(w, o[r].x, acc.x);
        acc.y = fmaf(w, o[r].y, acc.y);
        acc.z = fmaf(w, o[r].z, acc.z);
        acc.w = fmaf(w, o[r].w, acc.w);
      }
    }
    const float inv = (1.0f / ws) * unscale;   // times a power of two: exact
    out = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  store_y_nt(y + tok * kHeadDim + c4, out);
}

// Any number of rounds: a running softmax over the rounds, one round at a time.
template <typename T, bool O16, typename Y>
__global__ __launch_bounds__(256) void combine_many_kernel(
    const typename ORows<O16>::elem* __restrict__ o_rounds, const int32_t* __restrict__ hexp,
    const float* __restrict__ lse, const int32_t* __restrict__ inv_perm, const T* __restrict__ v,
    Y* __restrict__ y, int rounds, int L, int64_t total, int64_t blk0) {
  const int64_t tok0 = (blk0 + gridDim.x - 1 - blockIdx.x) * 16;
  const float unscale = o_unscale<O16>(hexp, tok0 / L);
  const int64_t tok = tok0 + (threadIdx.x >> 4);
  if (tok >= total) return;
  const int c4 = (threadIdx.x & 15) * 4;
  const int64_t bh = tok / L;
  const int i = (int)(tok % L);
  const int64_t seg0 = bh * rounds;
  float mx = -INFINITY;
  for (int r = 0; r < rounds; ++r) {
    const int64_t seg = seg0 + r;
    mx = fmaxf(mx, lse[seg * L + clamp_index(inv_perm[seg * L + i], L)]);
  }
  float4 out;
  if (mx == -INFINITY) {
    out = load_v4<T>(v + tok * kHeadDim, c4);
  } else {
    float ws = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < rounds; ++r) {
      const int64_t seg = seg0 + r;
      const int64_t row = seg * L + clamp_index(inv_perm[seg * L + i], L);
      const float w = expf(lse[row] - mx);
      const float4 o = ORows<O16>::load4(o_rounds + row * kHeadDim, c4);
      ws += w;
      acc.x = fmaf(w, o.x, acc.x);
      acc.y = fmaf(w, o.y, acc.y);
      acc.z = fmaf(w, o.z, acc.z);
      acc.w = fmaf(w, o.w, acc.w);
    }
    const float inv = (1.0f / ws) * unscale;
    out = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  store_y_nt(y + tok * kHeadDim + c4, out);
}

template <typename T, bool O16, typename Y>
static void launch_combine_t(const Shape& s, const void* o_buf, const float* lse,
                             const int32_t* inv_perm, const T* v, Y* y, hipStream_t stream) {
  const int32_t* hexp = reinterpret_cast<const int32_t*>(static_cast<const float*>(o_buf) +
                                                         (int64_t)s.batch * s.heads * kVParts);
  const auto* o_rounds = reinterpret_cast<const typename ORows<O16>::elem*>(
      static_cast<const char*>(o_buf) + o_header_bytes(s));
  const int64_t total = s.token_heads();
  const int64_t nblk = (total + 15) / 16;
  // pieces of at most kMaxBlocks workgroups, the last piece first (its
  // workgroups also run last-first)
  for (int64_t b0 = (nblk - 1) / kMaxBlocks * kMaxBlocks; b0 >= 0; b0 -= kMaxBlocks) {
    const dim3 grid((unsigned)std::min(kMaxBlocks, nblk - b0)), block(256);
#define LSH_COMBINE(K)                                                                       \
  hipLaunchKernelGGL(K, grid, block, 0, stream, o_rounds, hexp, lse, inv_perm, v, y, s.rounds, \
                     s.len, total, b0)
  if (s.rounds <= 1)
    LSH_COMBINE((combine_kernel<T, O16, 1, Y>));
  else if (s.rounds <= 2)
    LSH_COMBINE((combine_kernel<T, O16, 2, Y>));
  else if (s.rounds <= 4)
    LSH_COMBINE((combine_kernel<T, O16, 4, Y>));
  else if (s.rounds <= 8)
    LSH_COMBINE((combine_kernel<T, O16, 8, Y>));
  else if (s.rounds <= 16)
    LSH_COMBINE((combine_kernel<T, O16, 16, Y>));
  else
    LSH_COMBINE((combine_many_kernel<T, O16, Y>));
#undef LSH_COMBINE
  }
}

template <typename Y>
static hipError_t launch_combine_y(const Shape& s, const void* o_rounds, const float* lse,
                                   const int32_t* inv_perm, const void* v, Y* y,
                                   hipStream_t stream) {
  if (s.o16)
    launch_combine_t<uint16_t, true>(s, o_rounds, lse, inv_perm, static_cast<const uint16_t*>(v),
                                     y, stream);
  else if (s.bf16)
    launch_combine_t<uint16_t, false>(s, o_rounds, lse, inv_perm, static_cast<const uint16_t*>(v),
                                      y, stream);
  else
    launch_combine_t<float, false>(s, o_rounds, lse, inv_perm, static_cast<const float*>(v), y,
                                   stream);
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, const void* o_rounds, const float* lse,
                          const int32_t* inv_perm, const void* v, float* y, hipStream_t stream) {
  return launch_combine_y(s, o_rounds, lse, inv_perm, v, y, stream);
}

hipError_t launch_combine_bf16(const Shape& s, const void* o_rounds, const float* lse,
                               const int32_t* inv_perm, const void* v, uint16_t* y,
                               hipStream_t stream) {
  return launch_combine_y(s, o_rounds, lse, inv_perm, v, y, stream);
}

}  // namespace lsh
