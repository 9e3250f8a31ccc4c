// combine.hip -- unsort and combine the hash rounds (Reformer study note,
// section "Multiple Hash Rounds": the neighbourhood of a token is the union of
// its per-round neighbourhoods).  Taken as a multiset, the softmax over the
// union is the rounds' softmaxes merged with weights exp(lse_r - M) / sum.
//
// 16 lanes per token (4 features of the 64-wide row each); a 256-thread
// workgroup covers 16 consecutive tokens of one (batch, head), so y is written
// with full 256-byte rows while the per-round rows are gathered through
// inv_perm.  bf16 inputs: the per-round rows are fp16 of o * 2^-k with one k
// per (batch, head), recovered from the partial maxima of |v| in the header of
// the per-round buffer; 2^k is applied once, with the normalisation.
#include <math.h>

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

// Per-round rows, keyed by the input type T: fp32 rows for fp32 inputs, fp16
// rows for bf16 inputs (T = uint16_t).
template <typename T>
struct ORows;
template <>
struct ORows<float> {
  typedef float elem;
  __device__ static float4 load4(const float* row, int c4) {
    return *reinterpret_cast<const float4*>(row + c4);
  }
};
template <>
struct ORows<uint16_t> {
  typedef uint16_t elem;
  __device__ static float4 load4(const uint16_t* row, int c4) {
    const uint2 u = *reinterpret_cast<const uint2*>(row + c4);
    const half2v lo = __builtin_bit_cast(half2v, u.x), hi = __builtin_bit_cast(half2v, u.y);
    return make_float4((float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y);
  }
};

// 2^k of (batch, head) bh (1 for fp32 rows); every lane of the wave must call
// it.
template <typename T>
__device__ __forceinline__ float o_unscale(const float* vpart, int64_t bh) {
  if (sizeof(T) == sizeof(float)) return 1.0f;
  return pow2f(o_scale_exponent(head_vmax(vpart + bh * kVParts)));
}

// RMAX >= rounds: every round's slot, lse and output row are requested before
// any is used, so a token's R row gathers are in flight together.
template <typename T, int RMAX>
__global__ __launch_bounds__(256) void combine_kernel(
    const typename ORows<T>::elem* __restrict__ o_rounds, const float* __restrict__ vpart,
    const float* __restrict__ lse, const int32_t* __restrict__ inv_perm, const T* __restrict__ v,
    float* __restrict__ y, int rounds, int L, int64_t total) {
  // Last tokens first: the per-round rows written last by the attention step
  // are the likeliest to still sit in the memory-side cache.
  const int64_t tok0 = (int64_t)(gridDim.x - 1 - blockIdx.x) * 16;   // < total
  // the workgroup's 16 tokens lie in one (batch, head) (L is a multiple of 64)
  const float unscale = o_unscale<T>(vpart, tok0 / L);
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
    o[r] = ORows<T>::load4(o_rounds + row[r] * kHeadDim, c4);
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
  *reinterpret_cast<float4*>(y + tok * kHeadDim + c4) = out;
}

// Any number of rounds: a running softmax over the rounds, one round at a time.
template <typename T>
__global__ __launch_bounds__(256) void combine_many_kernel(
    const typename ORows<T>::elem* __restrict__ o_rounds, const float* __restrict__ vpart,
    const float* __restrict__ lse, const int32_t* __restrict__ inv_perm, const T* __restrict__ v,
    float* __restrict__ y, int rounds, int L, int64_t total) {
  const int64_t tok0 = (int64_t)(gridDim.x - 1 - blockIdx.x) * 16;
  const float unscale = o_unscale<T>(vpart, tok0 / L);
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
      const float4 o = ORows<T>::load4(o_rounds + row * kHeadDim, c4);
      ws += w;
      acc.x = fmaf(w, o.x, acc.x);
      acc.y = fmaf(w, o.y, acc.y);
      acc.z = fmaf(w, o.z, acc.z);
      acc.w = fmaf(w, o.w, acc.w);
    }
    const float inv = (1.0f / ws) * unscale;
    out = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  *reinterpret_cast<float4*>(y + tok * kHeadDim + c4) = out;
}

template <typename T>
static void launch_combine_t(const Shape& s, const void* o_buf, const float* lse,
                             const int32_t* inv_perm, const T* v, float* y, hipStream_t stream) {
  const float* vpart = static_cast<const float*>(o_buf);
  const auto* o_rounds = reinterpret_cast<const typename ORows<T>::elem*>(
      static_cast<const char*>(o_buf) + o_header_bytes(s));
  const int64_t total = s.token_heads();
  const dim3 grid((unsigned)((total + 15) / 16)), block(256);
#define LSH_COMBINE(K)                                                                       \
  hipLaunchKernelGGL(K, grid, block, 0, stream, o_rounds, vpart, lse, inv_perm, v, y, s.rounds, \
                     s.len, total)
  if (s.rounds <= 1)
    LSH_COMBINE((combine_kernel<T, 1>));
  else if (s.rounds <= 2)
    LSH_COMBINE((combine_kernel<T, 2>));
  else if (s.rounds <= 4)
    LSH_COMBINE((combine_kernel<T, 4>));
  else if (s.rounds <= 8)
    LSH_COMBINE((combine_kernel<T, 8>));
  else if (s.rounds <= 16)
    LSH_COMBINE((combine_kernel<T, 16>));
  else
    LSH_COMBINE(combine_many_kernel<T>);
#undef LSH_COMBINE
}

hipError_t launch_combine(const Shape& s, const void* o_rounds, const float* lse,
                          const int32_t* inv_perm, const void* v, float* y, hipStream_t stream) {
  if (s.bf16)
    launch_combine_t(s, o_rounds, lse, inv_perm, static_cast<const uint16_t*>(v), y, stream);
  else
    launch_combine_t(s, o_rounds, lse, inv_perm, static_cast<const float*>(v), y, stream);
  return hipGetLastError();
}

}  // namespace lsh
