// lsh_launch.h -- internal launchers of the gfx950 kernels (host side).
// The C ABI in api.hip validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lsh {

struct Shape {
  int batch, heads, len, buckets, rounds, causal, self_mask;
  bool bf16;   // qk, v, rot are bf16 (else fp32)
  bool o16;    // per-round outputs as fp16 rows with a per-(batch, head) scale (bf16 only)
  int64_t segments() const { return (int64_t)batch * heads * rounds; }
  int64_t token_heads() const { return (int64_t)batch * heads * len; }
};

hipError_t launch_hash(const Shape& s, const void* qk, const void* rot, int32_t* buckets,
                       uint32_t* fallback_rows, hipStream_t stream);
// Rotations [H][R][d][B/2] -> [H][R][B/2][d] (the rows launch_hash reads).
hipError_t launch_rot_rows(const Shape& s, const void* rot_cols, void* rot_rows,
                           hipStream_t stream);

// Sort tiling: each segment is cut into tiles of sort_tile(s) tokens.
int sort_tile(const Shape& s);
size_t sort_workspace_bytes(const Shape& s);
hipError_t launch_sort(const Shape& s, const int32_t* buckets, int32_t* perm, int32_t* inv_perm,
                       void* workspace, hipStream_t stream);
// The library's static device scratch for the sort: its size, and its device
// address on `device` (looked up on the first call for that device).
size_t static_sort_scratch_bytes();
hipError_t static_sort_scratch(int device, void** ptr);

// Per-round outputs.  fp32 rows [S][L][64] (any input dtype), or with o16: a
// header of kVParts partial maxima of |v| per (batch, head) (fp32) followed by
// the int32 scale exponent k of each (batch, head), padded to 256 bytes, then
// fp16 rows [S][L][64] holding o * 2^-k (o_scale_exponent of the head's
// maximum; kVParts and the rule are in lsh_device.h).
size_t o_header_bytes(const Shape& s);
size_t o_rounds_bytes(const Shape& s);

hipError_t launch_attend(const Shape& s, const void* qk, const void* v, const int32_t* buckets,
                         const int32_t* perm, void* o_rounds, float* lse, hipStream_t stream);

// Set union over rounds: workspace = per-token round keys (see attend.hip).
int union_key_stride(const Shape& s);
size_t union_workspace_bytes(const Shape& s);
hipError_t launch_attend_union(const Shape& s, const void* qk, const void* v,
                               const int32_t* buckets, const int32_t* perm,
                               const int32_t* inv_perm, void* o_rounds, float* lse,
                               void* workspace, hipStream_t stream);

hipError_t launch_combine(const Shape& s, const void* o_rounds, const float* lse,
                          const int32_t* inv_perm, const void* v, float* y, hipStream_t stream);
// the same with y rounded to bf16 (nearest even), for the reversible layer
hipError_t launch_combine_bf16(const Shape& s, const void* o_rounds, const float* lse,
                               const int32_t* inv_perm, const void* v, uint16_t* y,
                               hipStream_t stream);

hipError_t launch_local(const Shape& s, int before, int after, const void* qk, const void* v,
                        float* y, float* lse, hipStream_t stream);

// ------------------------------------------------ reversible layer (gemm.hip, layer.hip)
struct LayerShape {
  int batch, len, d_model, d_ff, ffn_chunk;   // heads = d_model / 64; ffn_chunk 0 = all rows
  int64_t rows() const { return (int64_t)batch * len; }
  int64_t chunk_rows() const { return ffn_chunk > 0 && ffn_chunk < rows() ? ffn_chunk : rows(); }
};

struct LayerWeights {
  const uint16_t *w_qk, *w_v, *w_o, *rot, *w_1, *w_2;
  const float *b_1, *b_2;
};

// qk, v [b][H][L][64] bf16 = bf16(bf16(x) W^T) for x fp32 [b*L][d_model]
hipError_t launch_project_qkv(const LayerShape& s, const float* x, const uint16_t* w_qk,
                              const uint16_t* w_v, uint16_t* qk, uint16_t* v, hipStream_t stream);
// out = resid + sign * (concat_heads(bf16(y_att)) W_o^T); out may equal resid
hipError_t launch_project_out(const LayerShape& s, const float* y_att, const uint16_t* w_o,
                              const float* resid, float sign, float* out, hipStream_t stream);
// the same with y_att already bf16 ([b][H][L][64])
hipError_t launch_project_out_bf16(const LayerShape& s, const uint16_t* y_att,
                                   const uint16_t* w_o, const float* resid, float sign,
                                   float* out, hipStream_t stream);
// out = resid + sign * (bf16(ReLU(bf16(x) W1^T + b1)) W2^T + b2), chunk by chunk of rows;
// hidden: chunk_rows() x d_ff bf16 scratch
hipError_t launch_ffn(const LayerShape& s, const float* x, const uint16_t* w_1, const float* b_1,
                      const uint16_t* w_2, const float* b_2, const float* resid, float sign,
                      float* out, uint16_t* hidden, hipStream_t stream);

size_t ffn_workspace_bytes(const LayerShape& s);
size_t layer_workspace_bytes(const LayerShape& ls, const Shape& as);
// forward: (y1, y2) = (x1 + F(x2), x2 + G(y1)); inverse: (x1, x2) from (y1, y2)
hipError_t launch_reversible(const LayerShape& ls, const Shape& as, const LayerWeights& w,
                             bool inverse, const float* in1, const float* in2, float* out1,
                             float* out2, void* workspace, hipStream_t stream);

}  // namespace lsh
