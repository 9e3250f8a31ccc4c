// lsh_launch.h -- internal launchers of the gfx950 kernels (host side).
// The C ABI in api.hip validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lsh {

struct Shape {
  int batch, heads, len, buckets, rounds, causal, self_mask;
  bool bf16;
  int64_t segments() const { return (int64_t)batch * heads * rounds; }
  int64_t token_heads() const { return (int64_t)batch * heads * len; }
};

hipError_t launch_hash(const Shape& s, const void* qk, const void* rot, int32_t* buckets,
                       uint32_t* fallback_rows, hipStream_t stream);

// Sort tiling: each segment is cut into tiles of sort_tile(s) tokens.
int sort_tile(const Shape& s);
size_t sort_workspace_bytes(const Shape& s);
hipError_t launch_sort(const Shape& s, const int32_t* buckets, int32_t* perm, int32_t* inv_perm,
                       void* workspace, hipStream_t stream);

hipError_t launch_attend(const Shape& s, const void* qk, const void* v, const int32_t* buckets,
                         const int32_t* perm, float* o_rounds, float* lse, hipStream_t stream);

// Set union over rounds: workspace = per-token round keys (see attend.hip).
int union_key_stride(const Shape& s);
size_t union_workspace_bytes(const Shape& s);
hipError_t launch_attend_union(const Shape& s, const void* qk, const void* v,
                               const int32_t* buckets, const int32_t* perm,
                               const int32_t* inv_perm, float* o_rounds, float* lse,
                               void* workspace, hipStream_t stream);

hipError_t launch_combine(const Shape& s, const float* o_rounds, const float* lse,
                          const int32_t* inv_perm, const void* v, float* y, hipStream_t stream);

hipError_t launch_local(const Shape& s, int before, int after, const void* qk, const void* v,
                        float* y, float* lse, hipStream_t stream);

}  // namespace lsh
