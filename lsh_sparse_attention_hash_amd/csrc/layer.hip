// layer.hip -- one reversible Reformer layer (Reformer study note, "Reversible
// Residual Layers"): y1 = x1 + F(x2), y2 = x2 + G(y1), and the inverse
// x2 = y2 - G(y1), x1 = y1 - F(x2).  F is the LSH attention of this library
// between two dense maps (qk and v projections, output projection); G is the
// chunked feed-forward map ("Chunked Feed-Forward Computation").  Host code
// only: it carves the caller's workspace and enqueues the kernels in order.
#include "lsh_device.h"
#include "lsh_launch.h"

namespace lsh {

namespace {

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct Carve {
  char* base;
  size_t at = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + at) : nullptr;
    at += align256(bytes);
    return p;
  }
};

struct LayerScratch {
  uint16_t *qk, *v, *hidden;
  int32_t *buckets, *perm, *inv_perm;
  void *sort_ws, *o_rounds;
  float* lse;
  uint16_t* y_att;   // bf16: the output map rounds its input to bf16 anyway
  size_t bytes;
};

LayerScratch carve(const LayerShape& ls, const Shape& as, void* base) {
  Carve c{static_cast<char*>(base)};
  LayerScratch w;
  const size_t T = (size_t)as.token_heads(), N = (size_t)as.segments() * as.len;
  w.qk = c.take<uint16_t>(T * kHeadDim * 2);
  w.v = c.take<uint16_t>(T * kHeadDim * 2);
  w.buckets = c.take<int32_t>(N * 4);
  w.perm = c.take<int32_t>(N * 4);
  w.inv_perm = c.take<int32_t>(N * 4);
  w.sort_ws = c.take<char>(sort_workspace_bytes(as));
  w.o_rounds = c.take<char>(o_rounds_bytes(as));
  w.lse = c.take<float>(N * 4);
  w.y_att = c.take<uint16_t>(T * kHeadDim * 2);
  w.hidden = c.take<uint16_t>(ffn_workspace_bytes(ls));
  w.bytes = c.at;
  return w;
}

// out = resid + sign * F(x)
hipError_t attention_block(const LayerShape& ls, const Shape& as, const LayerWeights& wt,
                           const LayerScratch& w, const float* x, const float* resid, float sign,
                           float* out, hipStream_t stream) {
  hipError_t e;
  if ((e = launch_project_qkv(ls, x, wt.w_qk, wt.w_v, w.qk, w.v, stream)) != hipSuccess) return e;
  if ((e = launch_hash(as, w.qk, wt.rot, w.buckets, nullptr, stream)) != hipSuccess) return e;
  if ((e = launch_sort(as, w.buckets, w.perm, w.inv_perm, w.sort_ws, stream)) != hipSuccess) return e;
  if ((e = launch_attend(as, w.qk, w.v, w.buckets, w.perm, w.o_rounds, w.lse, stream)) != hipSuccess)
    return e;
  if ((e = launch_combine_bf16(as, w.o_rounds, w.lse, w.inv_perm, w.v, w.y_att, stream)) !=
      hipSuccess)
    return e;
  return launch_project_out_bf16(ls, w.y_att, wt.w_o, resid, sign, out, stream);
}

}  // namespace

size_t ffn_workspace_bytes(const LayerShape& s) {
  return (size_t)s.chunk_rows() * s.d_ff * sizeof(uint16_t);
}

size_t layer_workspace_bytes(const LayerShape& ls, const Shape& as) {
  return carve(ls, as, nullptr).bytes;
}

hipError_t launch_reversible(const LayerShape& ls, const Shape& as, const LayerWeights& wt,
                             bool inverse, const float* in1, const float* in2, float* out1,
                             float* out2, void* workspace, hipStream_t stream) {
  const LayerScratch w = carve(ls, as, workspace);
  hipError_t e;
  if (!inverse) {
    // y1 = x1 + F(x2), then y2 = x2 + G(y1)
    if ((e = attention_block(ls, as, wt, w, in2, in1, 1.f, out1, stream)) != hipSuccess) return e;
    return launch_ffn(ls, out1, wt.w_1, wt.b_1, wt.w_2, wt.b_2, in2, 1.f, out2, w.hidden, stream);
  }
  // x2 = y2 - G(y1), then x1 = y1 - F(x2)
  if ((e = launch_ffn(ls, in1, wt.w_1, wt.b_1, wt.w_2, wt.b_2, in2, -1.f, out2, w.hidden,
                      stream)) != hipSuccess)
    return e;
  return attention_block(ls, as, wt, w, out2, in1, -1.f, out1, stream);
}

}  // namespace lsh
