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

lsh_status lsh_chunk_attend(const lsh_config* cfg, const void* qk, const void* v,
                            const int32_t* buckets, const int32_t* perm, float* o_rounds,
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

size_t lsh_union_workspace_bytes(const lsh_config* cfg) {
  lsh::Shape s;
  bool empty = false;
  if (check_config(cfg, &s, &empty) != LSH_OK || empty || check_union(s) != LSH_OK) return 0;
  return lsh::union_workspace_bytes(s);
}

lsh_status lsh_chunk_attend_union(const lsh_config* cfg, const void* qk, const void* v,
                                  const int32_t* buckets, const int32_t* perm,
                                  const int32_t* inv_perm, float* o_rounds, float* lse,
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

lsh_status lsh_unsort_combine(const lsh_config* cfg, const float* o_rounds, const float* lse,
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
