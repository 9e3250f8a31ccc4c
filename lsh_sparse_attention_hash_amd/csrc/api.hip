// api.hip -- the C ABI of liblsh (declared in include/lsh.h): argument
// validation on the host, then kernel launches on the caller's stream.
// Nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include "lsh.h"
#include "lsh_device.h"
#include "lsh_launch.h"

namespace {

thread_local char g_last_error[256] = "";

lsh_status fail(lsh_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

lsh_status ok() {
  g_last_error[0] = '\0';
  return LSH_OK;
}

// Validates cfg; fills s.  *empty is set for a problem with no tokens.
lsh_status check_config(const lsh_config* cfg, lsh::Shape* s, bool* empty) {
  if (!cfg) return fail(LSH_ERR_INVALID_ARGUMENT, "cfg is NULL");
  const lsh_config& c = *cfg;
  if (c.batch < 0 || c.heads < 0 || c.seq_len < 0)
    return fail(LSH_ERR_INVALID_ARGUMENT, "negative batch/heads/seq_len");
  if (c.dtype != LSH_F32 && c.dtype != LSH_BF16)
    return fail(LSH_ERR_INVALID_ARGUMENT, "dtype %d is not LSH_F32 or LSH_BF16", c.dtype);
  if (c.n_buckets < 1 || c.n_buckets > 16384 || (c.n_buckets > 1 && (c.n_buckets & 1)))
    return fail(LSH_ERR_INVALID_ARGUMENT, "n_buckets %d must be 1 or even in [2, 16384]",
                c.n_buckets);
  if (c.n_rounds < 1 || c.n_rounds > 1024)
    return fail(LSH_ERR_INVALID_ARGUMENT, "n_rounds %d outside [1, 1024]", c.n_rounds);
  if ((c.causal != 0 && c.causal != 1) || (c.self_mask != 0 && c.self_mask != 1))
    return fail(LSH_ERR_INVALID_ARGUMENT, "causal and self_mask must be 0 or 1");
  if (c.o_format != LSH_O_F32 && c.o_format != LSH_O_F16_SCALED)
    return fail(LSH_ERR_INVALID_ARGUMENT, "o_format %d is not LSH_O_F32 or LSH_O_F16_SCALED",
                c.o_format);
  if (c.o_format == LSH_O_F16_SCALED && c.dtype != LSH_BF16)
    return fail(LSH_ERR_UNSUPPORTED, "LSH_O_F16_SCALED needs bf16 inputs");
  if (c.head_dim != lsh::kHeadDim)
    return fail(LSH_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", c.head_dim);
  if (c.chunk_len != lsh::kChunk)
    return fail(LSH_ERR_UNSUPPORTED, "chunk_len %d unsupported (only 64)", c.chunk_len);
  *empty = c.batch == 0 || c.heads == 0 || c.seq_len == 0;
  if (!*empty) {
    if (c.seq_len % c.chunk_len)
      return fail(LSH_ERR_INVALID_ARGUMENT, "seq_len %d is not a multiple of chunk_len %d",
                  c.seq_len, c.chunk_len);
    const long long rows = (long long)c.batch * c.heads * c.n_rounds * c.seq_len;
    if (rows >= (1LL << 31))
      return fail(LSH_ERR_INVALID_ARGUMENT, "batch*heads*n_rounds*seq_len = %lld >= 2^31", rows);
    if (c.batch > 65535 || c.heads > 65535)
      return fail(LSH_ERR_INVALID_ARGUMENT, "batch and heads must be <= 65535");
  }
  s->batch = c.batch;
  s->heads = c.heads;
  s->len = c.seq_len;
  s->buckets = c.n_buckets;
  s->rounds = c.n_rounds;
  s->causal = c.causal;
  s->self_mask = c.self_mask;
  s->bf16 = c.dtype == LSH_BF16;
  s->o16 = c.o_format == LSH_O_F16_SCALED;
  return LSH_OK;
}

lsh_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(LSH_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & 15)
    return fail(LSH_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return LSH_OK;
}

lsh_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LSH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Shapes the set-union attention supports (beyond check_config).
lsh_status check_union(const lsh::Shape& s) {
  if (s.rounds > 16)
    return fail(LSH_ERR_UNSUPPORTED, "set union supports n_rounds <= 16 (got %d)", s.rounds);
  const long long span = (long long)s.len / lsh::kChunk + 1;
  if ((long long)s.buckets * span >= (1LL << 31))
    return fail(LSH_ERR_UNSUPPORTED, "set union needs n_buckets * (seq_len / 64 + 1) < 2^31");
  return LSH_OK;
}

#define LSH_TRY(expr)                 \
  do {                                \
    const lsh_status st_ = (expr);    \
    if (st_ != LSH_OK) return st_;    \
  } while (0)

// Validates a layer configuration; fills the layer shape and the shape of its
// attention (bf16, head_dim = chunk_len = 64).  *empty: no tokens.
lsh_status check_layer(const lsh_layer_config* cfg, lsh::LayerShape* ls, lsh::Shape* as,
                       bool* empty) {
  if (!cfg) return fail(LSH_ERR_INVALID_ARGUMENT, "cfg is NULL");
  const lsh_layer_config& c = *cfg;
  if (c.d_model < lsh::kHeadDim || c.d_model % lsh::kHeadDim)
    return fail(LSH_ERR_UNSUPPORTED, "d_model %d must be a positive multiple of 64", c.d_model);
  if (c.d_ff < 64 || c.d_ff % 64)
    return fail(LSH_ERR_UNSUPPORTED, "d_ff %d must be a positive multiple of 64", c.d_ff);
  if (c.ffn_chunk < 0) return fail(LSH_ERR_INVALID_ARGUMENT, "ffn_chunk %d < 0", c.ffn_chunk);
  lsh_config a;
  a.batch = c.batch;
  a.heads = c.d_model / lsh::kHeadDim;
  a.seq_len = c.seq_len;
  a.head_dim = lsh::kHeadDim;
  a.n_buckets = c.n_buckets;
  a.n_rounds = c.n_rounds;
  a.chunk_len = lsh::kChunk;
  a.causal = c.causal;
  a.self_mask = c.self_mask;
  a.dtype = LSH_BF16;
  a.o_format = LSH_O_F16_SCALED;   // the layer's own intermediate, half the bytes
  LSH_TRY(check_config(&a, as, empty));
  const long long rows = (long long)c.batch * c.seq_len;
  if (rows * (c.d_model > c.d_ff ? c.d_model : c.d_ff) >= (1LL << 40))
    return fail(LSH_ERR_INVALID_ARGUMENT, "batch*seq_len*max(d_model, d_ff) too large");
  ls->batch = c.batch;
  ls->len = c.seq_len;
  ls->d_model = c.d_model;
  ls->d_ff = c.d_ff;
  ls->ffn_chunk = c.ffn_chunk;
  return LSH_OK;
}

}  // namespace

extern "C" {

lsh_status lsh_hash(const lsh_config* cfg, const void* qk, const void* rot, int32_t* buckets,
                    uint32_t* fallback_rows, void* stream) {
  lsh::Shape s;
  bool empty = false;
  LSH_TRY(check_config(cfg, &s, &empty));
  if (empty) return ok();
  LSH_TRY(check_ptr(qk, "qk"));
  if (s.buckets > 1) LSH_TRY(check_ptr(rot, "rot"));
  LSH_TRY(check_ptr(buckets, "buckets"));
  if (fallback_rows && (reinterpret_cast<uintptr_t>(fallback_rows) & 3))
    return fail(LSH_ERR_INVALID_ARGUMENT, "fallback_rows is not 4-byte aligned");
  return launched(lsh::launch_hash(s, qk, rot, buckets, fallback_rows,
                                   static_cast<hipStream_t>(stream)),
                  "lsh_hash");
}

lsh_status lsh_rot_from_columns(const lsh_config* cfg, const void* rot_cols, void* rot_rows,
                                void* stream) {
  lsh::Shape s;
  bool empty = false;
  LSH_TRY(check_config(cfg, &s, &empty));
  if (s.heads == 0 || s.buckets == 1) return ok();   // no rotation to convert
  LSH_TRY(check_ptr(rot_cols, "rot_cols"));
  LSH_TRY(check_ptr(rot_rows, "rot_rows"));
  const size_t bytes = (size_t)s.heads * s.rounds * (s.buckets / 2) * lsh::kHeadDim *
                       (s.bf16 ? sizeof(uint16_t) : sizeof(float));
  const uintptr_t a = reinterpret_cast<uintptr_t>(rot_cols), b = reinterpret_cast<uintptr_t>(rot_rows);
  if (a < b + bytes && b < a + bytes)
    return fail(LSH_ERR_INVALID_ARGUMENT, "rot_cols and rot_rows overlap");
  return launched(lsh::launch_rot_rows(s, rot_cols, rot_rows, static_cast<hipStream_t>(stream)),
                  "lsh_rot_from_columns");
}

size_t lsh_sort_workspace_bytes(const lsh_config* cfg) {
  lsh::Shape s;
  bool empty = false;
  if (check_config(cfg, &s, &empty) != LSH_OK || empty) return 0;
  return lsh::sort_workspace_bytes(s);
}

lsh_status lsh_sort(const lsh_config* cfg, const int32_t* buckets, int32_t* perm,
                    int32_t* inv_perm, void* workspace, size_t workspace_bytes, void* stream) {
  lsh::Shape s;
  bool empty = false;
  LSH_TRY(check_config(cfg, &s, &empty));
  if (empty) return ok();
  LSH_TRY(check_ptr(buckets, "buckets"));
  LSH_TRY(check_ptr(perm, "perm"));
  LSH_TRY(check_ptr(inv_perm, "inv_perm"));
  LSH_TRY(check_ptr(workspace, "workspace"));
  const size_t need = lsh::sort_workspace_bytes(s);
  if (workspace_bytes < need)
    return fail(LSH_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed",
                workspace_bytes, need);
  return launched(lsh::launch_sort(s, buckets, perm, inv_perm, workspace,
                                   static_cast<hipStream_t>(stream)),
                  "lsh_sort");
}

lsh_status lsh_sort_static_scratch(const lsh_config* cfg, const int32_t* buckets,
                                   int32_t* perm, int32_t* inv_perm, void* stream) {
  lsh::Shape s;
  bool empty = false;
  LSH_TRY(check_config(cfg, &s, &empty));
  if (empty) return ok();
  LSH_TRY(check_ptr(buckets, "buckets"));
  LSH_TRY(check_ptr(perm, "perm"));
  LSH_TRY(check_ptr(inv_perm, "inv_perm"));
  const size_t need = lsh::sort_workspace_bytes(s);
  if (need > lsh::static_sort_scratch_bytes())
    return fail(LSH_ERR_WORKSPACE_TOO_SMALL,
                "the sort needs %zu bytes of scratch, the static scratch holds %zu", need,
                lsh::static_sort_scratch_bytes());
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int device = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &device) : hipGetDevice(&device);
  if (e != hipSuccess) return launched(e, "lsh_sort_static_scratch: device of the stream");
  void* ws = nullptr;
  e = lsh::static_sort_scratch(device, &ws);
  if (e != hipSuccess) return launched(e, "lsh_sort_static_scratch: scratch address");
  return launched(lsh::launch_sort(s, buckets, perm, inv_perm, ws, st), "lsh_sort_static_scratch");
}

lsh_status lsh_chunk_attend(const lsh_config* cfg, const void* qk, const void* v,
                            const int32_t* buckets, const int32_t* perm, void* o_rounds,
                            float* lse, void* stream) {
  lsh::Shape s;
  bool empty = false;
  LSH_TRY(check_config(cfg, &s, &empty));
  if (empty) return ok();
  LSH_TRY(check_ptr(qk, "qk"));
  LSH_TRY(check_ptr(v, "v"));
  LSH_TRY(check_ptr(buckets, "buckets"));
  LSH_TRY(check_ptr(perm, "perm"));
  LSH_TRY(check_ptr(o_rounds, "o_rounds"));
  LSH_TRY(check_ptr(lse, "lse"));
  return launched(lsh::launch_attend(s, qk, v, buckets, perm, o_rounds, lse,
                                     static_cast<hipStream_t>(stream)),
                  "lsh_chunk_attend");
}

size_t lsh_o_rounds_bytes(const lsh_config* cfg) {
  lsh::Shape s;
  bool empty = false;
  if (check_config(cfg, &s, &empty) != LSH_OK || empty) return 0;
  return lsh::o_rounds_bytes(s);
}

size_t lsh_union_workspace_bytes(const lsh_config* cfg) {
  lsh::Shape s;
  bool empty = false;
  if (check_config(cfg, &s, &empty) != LSH_OK || empty || check_union(s) != LSH_OK) return 0;
  return lsh::union_workspace_bytes(s);
}

lsh_status lsh_chunk_attend_union(const lsh_config* cfg, const void* qk, const void* v,
                                  const int32_t* buckets, const int32_t* perm,
                                  const int32_t* inv_perm, void* o_rounds, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  lsh::Shape s;
  bool empty = false;
  LSH_TRY(check_config(cfg, &s, &empty));
  if (empty) return ok();
  LSH_TRY(check_union(s));
  LSH_TRY(check_ptr(qk, "qk"));
  LSH_TRY(check_ptr(v, "v"));
  LSH_TRY(check_ptr(buckets, "buckets"));
  LSH_TRY(check_ptr(perm, "perm"));
  LSH_TRY(check_ptr(inv_perm, "inv_perm"));
  LSH_TRY(check_ptr(o_rounds, "o_rounds"));
  LSH_TRY(check_ptr(lse, "lse"));
  LSH_TRY(check_ptr(workspace, "workspace"));
  const size_t need = lsh::union_workspace_bytes(s);
  if (workspace_bytes < need)
    return fail(LSH_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed",
                workspace_bytes, need);
  return launched(lsh::launch_attend_union(s, qk, v, buckets, perm, inv_perm, o_rounds, lse,
                                           workspace, static_cast<hipStream_t>(stream)),
                  "lsh_chunk_attend_union");
}

lsh_status lsh_unsort_combine(const lsh_config* cfg, const void* o_rounds, const float* lse,
                              const int32_t* inv_perm, const void* v, float* y, void* stream) {
  lsh::Shape s;
  bool empty = false;
  LSH_TRY(check_config(cfg, &s, &empty));
  if (empty) return ok();
  LSH_TRY(check_ptr(o_rounds, "o_rounds"));
  LSH_TRY(check_ptr(lse, "lse"));
  LSH_TRY(check_ptr(inv_perm, "inv_perm"));
  LSH_TRY(check_ptr(v, "v"));
  LSH_TRY(check_ptr(y, "y"));
  return launched(lsh::launch_combine(s, o_rounds, lse, inv_perm, v, y,
                                      static_cast<hipStream_t>(stream)),
                  "lsh_unsort_combine");
}

lsh_status lsh_local_attend(const lsh_config* cfg, int32_t n_before, int32_t n_after,
                            const void* qk, const void* v, float* y, float* lse, void* stream) {
  if (!cfg) return fail(LSH_ERR_INVALID_ARGUMENT, "cfg is NULL");
  // no hashing: the bucket and round fields are not used
  lsh_config c = *cfg;
  c.n_buckets = 1;
  c.n_rounds = 1;
  lsh::Shape s;
  bool empty = false;
  LSH_TRY(check_config(&c, &s, &empty));
  if (n_before < 0 || n_after < 0)
    return fail(LSH_ERR_INVALID_ARGUMENT, "n_before %d and n_after %d must be >= 0", n_before,
                n_after);
  if (empty) return ok();
  LSH_TRY(check_ptr(qk, "qk"));
  LSH_TRY(check_ptr(v, "v"));
  LSH_TRY(check_ptr(y, "y"));
  LSH_TRY(check_ptr(lse, "lse"));
  return launched(lsh::launch_local(s, n_before, n_after, qk, v, y, lse,
                                    static_cast<hipStream_t>(stream)),
                  "lsh_local_attend");
}

lsh_status lsh_project_qkv(const lsh_layer_config* cfg, const float* x, const void* w_qk,
                           const void* w_v, void* qk, void* v, void* stream) {
  lsh::LayerShape ls;
  lsh::Shape as;
  bool empty = false;
  LSH_TRY(check_layer(cfg, &ls, &as, &empty));
  if (empty) return ok();
  LSH_TRY(check_ptr(x, "x"));
  LSH_TRY(check_ptr(w_qk, "w_qk"));
  LSH_TRY(check_ptr(w_v, "w_v"));
  LSH_TRY(check_ptr(qk, "qk"));
  LSH_TRY(check_ptr(v, "v"));
  return launched(lsh::launch_project_qkv(ls, x, static_cast<const uint16_t*>(w_qk),
                                          static_cast<const uint16_t*>(w_v),
                                          static_cast<uint16_t*>(qk), static_cast<uint16_t*>(v),
                                          static_cast<hipStream_t>(stream)),
                  "lsh_project_qkv");
}

lsh_status lsh_project_out(const lsh_layer_config* cfg, const float* y_att, const void* w_o,
                           const float* resid, int32_t subtract, float* out, void* stream) {
  lsh::LayerShape ls;
  lsh::Shape as;
  bool empty = false;
  LSH_TRY(check_layer(cfg, &ls, &as, &empty));
  if (subtract != 0 && subtract != 1)
    return fail(LSH_ERR_INVALID_ARGUMENT, "subtract must be 0 or 1");
  if (empty) return ok();
  LSH_TRY(check_ptr(y_att, "y_att"));
  LSH_TRY(check_ptr(w_o, "w_o"));
  LSH_TRY(check_ptr(resid, "resid"));
  LSH_TRY(check_ptr(out, "out"));
  return launched(lsh::launch_project_out(ls, y_att, static_cast<const uint16_t*>(w_o), resid,
                                          subtract ? -1.f : 1.f, out,
                                          static_cast<hipStream_t>(stream)),
                  "lsh_project_out");
}

size_t lsh_ffn_workspace_bytes(const lsh_layer_config* cfg) {
  lsh::LayerShape ls;
  lsh::Shape as;
  bool empty = false;
  if (check_layer(cfg, &ls, &as, &empty) != LSH_OK || empty) return 0;
  return lsh::ffn_workspace_bytes(ls);
}

lsh_status lsh_ffn(const lsh_layer_config* cfg, const float* x, const void* w_1, const float* b_1,
                   const void* w_2, const float* b_2, const float* resid, int32_t subtract,
                   float* out, void* workspace, size_t workspace_bytes, void* stream) {
  lsh::LayerShape ls;
  lsh::Shape as;
  bool empty = false;
  LSH_TRY(check_layer(cfg, &ls, &as, &empty));
  if (subtract != 0 && subtract != 1)
    return fail(LSH_ERR_INVALID_ARGUMENT, "subtract must be 0 or 1");
  if (empty) return ok();
  LSH_TRY(check_ptr(x, "x"));
  LSH_TRY(check_ptr(w_1, "w_1"));
  LSH_TRY(check_ptr(b_1, "b_1"));
  LSH_TRY(check_ptr(w_2, "w_2"));
  LSH_TRY(check_ptr(b_2, "b_2"));
  LSH_TRY(check_ptr(resid, "resid"));
  LSH_TRY(check_ptr(out, "out"));
  LSH_TRY(check_ptr(workspace, "workspace"));
  const size_t need = lsh::ffn_workspace_bytes(ls);
  if (workspace_bytes < need)
    return fail(LSH_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed",
                workspace_bytes, need);
  return launched(lsh::launch_ffn(ls, x, static_cast<const uint16_t*>(w_1), b_1,
                                  static_cast<const uint16_t*>(w_2), b_2, resid,
                                  subtract ? -1.f : 1.f, out, static_cast<uint16_t*>(workspace),
                                  static_cast<hipStream_t>(stream)),
                  "lsh_ffn");
}

size_t lsh_layer_workspace_bytes(const lsh_layer_config* cfg) {
  lsh::LayerShape ls;
  lsh::Shape as;
  bool empty = false;
  if (check_layer(cfg, &ls, &as, &empty) != LSH_OK || empty) return 0;
  return lsh::layer_workspace_bytes(ls, as);
}

static lsh_status reversible(const char* name, bool inverse, const lsh_layer_config* cfg,
                             const lsh_layer_weights* w, const float* in1, const float* in2,
                             float* out1, float* out2, void* workspace, size_t workspace_bytes,
                             void* stream) {
  lsh::LayerShape ls;
  lsh::Shape as;
  bool empty = false;
  LSH_TRY(check_layer(cfg, &ls, &as, &empty));
  if (empty) return ok();
  if (!w) return fail(LSH_ERR_INVALID_ARGUMENT, "weights is NULL");
  LSH_TRY(check_ptr(w->w_qk, "w_qk"));
  LSH_TRY(check_ptr(w->w_v, "w_v"));
  LSH_TRY(check_ptr(w->w_o, "w_o"));
  if (as.buckets > 1) LSH_TRY(check_ptr(w->rot, "rot"));
  LSH_TRY(check_ptr(w->w_1, "w_1"));
  LSH_TRY(check_ptr(w->b_1, "b_1"));
  LSH_TRY(check_ptr(w->w_2, "w_2"));
  LSH_TRY(check_ptr(w->b_2, "b_2"));
  LSH_TRY(check_ptr(in1, "first input"));
  LSH_TRY(check_ptr(in2, "second input"));
  LSH_TRY(check_ptr(out1, "first output"));
  LSH_TRY(check_ptr(out2, "second output"));
  LSH_TRY(check_ptr(workspace, "workspace"));
  const size_t need = lsh::layer_workspace_bytes(ls, as);
  if (workspace_bytes < need)
    return fail(LSH_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed",
                workspace_bytes, need);
  lsh::LayerWeights lw;
  lw.w_qk = static_cast<const uint16_t*>(w->w_qk);
  lw.w_v = static_cast<const uint16_t*>(w->w_v);
  lw.w_o = static_cast<const uint16_t*>(w->w_o);
  lw.rot = static_cast<const uint16_t*>(w->rot);
  lw.w_1 = static_cast<const uint16_t*>(w->w_1);
  lw.b_1 = w->b_1;
  lw.w_2 = static_cast<const uint16_t*>(w->w_2);
  lw.b_2 = w->b_2;
  return launched(lsh::launch_reversible(ls, as, lw, inverse, in1, in2, out1, out2, workspace,
                                         static_cast<hipStream_t>(stream)),
                  name);
}

lsh_status lsh_reversible_forward(const lsh_layer_config* cfg, const lsh_layer_weights* w,
                                  const float* x1, const float* x2, float* y1, float* y2,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return reversible("lsh_reversible_forward", false, cfg, w, x1, x2, y1, y2, workspace,
                    workspace_bytes, stream);
}

lsh_status lsh_reversible_inverse(const lsh_layer_config* cfg, const lsh_layer_weights* w,
                                  const float* y1, const float* y2, float* x1, float* x2,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return reversible("lsh_reversible_inverse", true, cfg, w, y1, y2, x1, x2, workspace,
                    workspace_bytes, stream);
}

const char* lsh_status_string(lsh_status status) {
  switch (status) {
    case LSH_OK: return "ok";
    case LSH_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LSH_ERR_UNSUPPORTED: return "unsupported shape";
    case LSH_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LSH_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

const char* lsh_last_error(void) { return g_last_error; }

int lsh_version(void) { return 10000; }

}  // extern "C"
