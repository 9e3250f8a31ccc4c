/*
 * lsh.h -- C ABI of the MI355X (gfx950) LSH-attention forward library,
 * liblsh.so.
 *
 * The library computes the forward pass of Reformer's LSH attention (Kitaev,
 * Kaiser, Levskaya, "Reformer: The Efficient Transformer", ICLR 2020) as four
 * calls that follow the pipeline the Reformer study note
 * (eightmm.github.io/papers/architectures/reformer) states in its section
 * "Sorting and Chunking":
 *
 *     X --hash--> bucket ids --sort--> bucket-contiguous sequence
 *       --chunked attention--> per-round outputs --unsort + combine--> Y
 *
 * Notation: batch b, heads H, sequence length L, head dim d, buckets B,
 * rounds R, chunk length m.  A "segment" is one (batch, head, round) triple,
 * numbered seg = (b_idx * H + h) * R + r.  x_i is the shared query/key vector
 * of token i (Q = K, note section "Shared Query-Key Space"), v_i its value.
 *
 * Conventions shared by every call
 *   - Every tensor is dense, row-major and lives in device memory owned by the
 *     caller; the library never allocates device memory and keeps no state
 *     between calls.  Device pointers must be 16-byte aligned.
 *   - Every call is asynchronous: it validates its arguments on the host,
 *     enqueues its kernels on `stream` (a hipStream_t; NULL = the default
 *     stream) and returns.  The caller synchronises.
 *   - Argument errors are detected on the host before anything is enqueued,
 *     so an error leaves every output untouched.  A failed launch returns
 *     LSH_ERR_HIP.  lsh_last_error() describes the last failure of the
 *     calling thread.
 *   - Supported shapes: head_dim == 64 and chunk_len == 64 (else
 *     LSH_ERR_UNSUPPORTED); seq_len a multiple of chunk_len; n_buckets 1 or
 *     even with 2 <= n_buckets <= 16384; 1 <= n_rounds <= 1024;
 *     batch * heads * n_rounds * seq_len < 2^31.  A zero batch, heads or
 *     seq_len is an empty problem: the call returns LSH_OK and does nothing.
 *   - Inputs must be finite, with |x|_2 < 2^60 and |R_j|_2 < 2^60 (the
 *     fp32 headroom of the matrix-core scores and the squared key norms).
 *   - Calls are thread-safe and may run concurrently on different streams.
 */
#ifndef LSH_H_
#define LSH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LSH_OK = 0,
  LSH_ERR_INVALID_ARGUMENT = 1,
  LSH_ERR_UNSUPPORTED = 2,
  LSH_ERR_WORKSPACE_TOO_SMALL = 3,
  LSH_ERR_HIP = 4
} lsh_status;

typedef enum { LSH_F32 = 0, LSH_BF16 = 1 } lsh_dtype;

/* Storage of the per-round outputs o between lsh_chunk_attend and
 * lsh_unsort_combine (the layouts are given at lsh_chunk_attend). */
typedef enum {
  LSH_O_F32 = 0,        /* fp32 rows, for either input dtype (the default) */
  LSH_O_F16_SCALED = 1  /* bf16 inputs only: fp16 rows with one power-of-two
                           scale per (batch, head), half the bytes */
} lsh_o_format;

typedef struct {
  int32_t batch;     /* b */
  int32_t heads;     /* H */
  int32_t seq_len;   /* L */
  int32_t head_dim;  /* d (64) */
  int32_t n_buckets; /* B: 1 (no hashing, every token in bucket 0) or even */
  int32_t n_rounds;  /* R: independent hash rounds */
  int32_t chunk_len; /* m (64) */
  int32_t causal;    /* 1: key j is masked for query i when j > i (original positions) */
  int32_t self_mask; /* 1: a token is never its own key; if no round leaves it
                        any key, its output is its own value */
  int32_t dtype;     /* lsh_dtype of qk, v and rot */
  int32_t o_format;  /* lsh_o_format of the per-round outputs (0 = fp32 rows);
                        LSH_O_F16_SCALED with fp32 inputs is LSH_ERR_UNSUPPORTED */
} lsh_config;

/*
 * lsh_hash -- angular LSH bucket of every token in every round.
 * Follows: Reformer study note, section "LSH Attention" (a hash h(x) into B
 * buckets under which similar vectors collide more often), realised as the
 * random-rotation angular hash; "Multiple Hash Rounds" (R independent hashes).
 *
 *   qk       [b][H][L][d]      dtype  shared query/key vectors x
 *   rot      [H][R][B/2][d]    dtype  rotation of head h, round r stored as
 *                                     B/2 direction rows: rot[h][r][j][k] is
 *                                     R_{h,r}[k][j].  May be NULL if B == 1.
 *   buckets  [b][H][R][L]      int32  output, original token order
 *   fallback_rows  optional device uint32 counter (NULL = not wanted).  The
 *            call ADDS the number of (token, round) rows whose bucket it
 *            decided by exact fp64 recomputation because the fast matrix-core
 *            scores could not separate the two best candidates.
 *
 * bucket = the 0-based index of the largest entry of the B-vector
 * [x R ; -(x R)], lowest index on ties, where x R is defined as the fp64 sum
 * over k = 0..d-1 taken in that order.  The result equals that definition
 * bit for bit: bf16 inputs are scored on the matrix cores with fp32
 * accumulation and every row whose margin is within the proven rounding bound
 * is recomputed in fp64 in the defining order; fp32 inputs are scored in fp64.
 * B == 1: every bucket is 0.
 */
lsh_status lsh_hash(const lsh_config* cfg, const void* qk, const void* rot,
                    int32_t* buckets, uint32_t* fallback_rows, void* stream);

/*
 * lsh_rot_from_columns -- rotations stored as d x B/2 matrices, rewritten as
 * the direction rows lsh_hash reads.
 * Follows: Reformer study note, section "LSH Attention" (the random-rotation
 * hash; R_{h,r} is a d x B/2 matrix applied to x).
 *
 *   rot_cols  [H][R][d][B/2]   dtype  input:  rot_cols[h][r][k][j] = R_{h,r}[k][j]
 *   rot_rows  [H][R][B/2][d]   dtype  output: rot_rows[h][r][j][k] = R_{h,r}[k][j]
 *
 * A transposition of every (head, round) matrix, bits unchanged, enqueued on
 * `stream`.  Uses cfg's heads, n_rounds, n_buckets, head_dim and dtype (the
 * other fields must still form a valid configuration; batch and seq_len may be
 * 0).  Both buffers are device memory owned by the caller, 16-byte aligned,
 * and must not overlap (LSH_ERR_INVALID_ARGUMENT).  Nothing to do (LSH_OK,
 * pointers unused) when heads == 0 or n_buckets == 1.  Rotations are
 * parameters: convert them once and pass rot_rows to every lsh_hash call.
 */
lsh_status lsh_rot_from_columns(const lsh_config* cfg, const void* rot_cols, void* rot_rows,
                                void* stream);

/* Bytes of device workspace lsh_sort needs for cfg (0 for an empty problem). */
size_t lsh_sort_workspace_bytes(const lsh_config* cfg);

/*
 * lsh_sort -- stable sort of every segment by bucket.
 * Follows: Reformer study note, section "Sorting and Chunking" (tokens are
 * sorted by hash bucket so that each bucket is contiguous).
 *
 *   buckets   [b][H][R][L] int32 in [0, B)     input (from lsh_hash)
 *   perm      [b][H][R][L] int32               output: perm[seg][s] is the
 *                                              original position at sorted slot s
 *   inv_perm  [b][H][R][L] int32               output: inv_perm[seg][perm[seg][s]] = s
 *   workspace device scratch of at least lsh_sort_workspace_bytes(cfg) bytes
 *             (else LSH_ERR_WORKSPACE_TOO_SMALL); contents on entry ignored.
 *
 * Sorted order is by the unique key (bucket, original position), so the
 * result is unique.  Bucket ids outside [0, B) are clamped into range (the
 * outputs are then still permutations, but the order is unspecified).
 */
lsh_status lsh_sort(const lsh_config* cfg, const int32_t* buckets,
                    int32_t* perm, int32_t* inv_perm, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * lsh_sort_static_scratch -- lsh_sort without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid allocation).
 *
 *   cfg, buckets, perm, inv_perm   as for lsh_sort
 *
 * Same results as lsh_sort.  The count tables live in a static array of
 * 32 MiB of device memory inside the library, one per GPU, held until the
 * process ends; nothing is allocated by the call.  A configuration whose
 * lsh_sort_workspace_bytes(cfg) exceeds 32 MiB returns
 * LSH_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  Every call on one
 * GPU shares that GPU's array: calls that may overlap on one GPU (different
 * streams, or different threads) race and must be serialised by the caller.
 * The array's address on a GPU is looked up on the first call there.
 */
lsh_status lsh_sort_static_scratch(const lsh_config* cfg, const int32_t* buckets,
                                   int32_t* perm, int32_t* inv_perm, void* stream);

/*
 * lsh_chunk_attend -- attention inside chunks of the bucket-sorted sequence.
 * Follows: Reformer study note, sections "LSH Attention" (candidate set
 * N_LSH(i) = same-bucket keys; y_i = softmax-weighted sum of v_j over it with
 * scores q_i.k_j / sqrt(d)), "Shared Query-Key Space" (Q = K), "Sorting and
 * Chunking" (attention over chunks of nearby sorted positions) and
 * "Implementation Reading" (causal masking by original position; same-token
 * policy).
 *
 *   qk, v     [b][H][L][d]        dtype
 *   buckets   [b][H][R][L]        int32, original order (from lsh_hash)
 *   perm      [b][H][R][L]        int32 (from lsh_sort)
 *   o_rounds  device buffer of lsh_o_rounds_bytes(cfg) bytes (see below):
 *             the per-round outputs o, SORTED order
 *   lse       [b][H][R][L]        fp32 output, SORTED order
 *
 * For the query i = perm[seg][s] of sorted chunk c = s / m, the window is the
 * slots of chunks c-1 (if c > 0) and c.  Its keys are the tokens j of the
 * window with bucket_j == bucket_i, j <= i if causal, and j != i if
 * self_mask.  With s_ij = (x_i . x_j) / (max(|x_j|_2, 1e-6) * sqrt(d)):
 *   lse[seg][s] = log sum_j exp(s_ij)           (-inf if there is no key)
 *   o_rounds[seg][s] = sum_j exp(s_ij - lse) v_j  (0 if there is no key)
 * bf16 inputs use bf16 matrix-core products with fp32 accumulation; fp32
 * inputs use fp32 arithmetic.
 *
 * Layout of o_rounds (written here, read by lsh_unsort_combine), chosen by
 * cfg->o_format:
 *   LSH_O_F32: o as fp32 [b][H][R][L][d] (bf16 or fp32 inputs).
 *   LSH_O_F16_SCALED (bf16 inputs): a header of 256 fp32 partial maxima of
 *     |v| per (b, h) ([b][H][256]) followed by the int32 exponent k of each
 *     (b, h) ([b][H]), padded to a multiple of 256 bytes, then o as fp16
 *     [b][H][R][L][d] holding o * 2^-k (round to nearest even).  With V the
 *     largest of the (b, h)'s 256 partial maxima and e the smallest integer
 *     with V < 2^e (e = -126 when V < 2^-126), k = max(e - 15, -100).
 *     Each o is a weighted mean of v rows, so every stored |o| * 2^-k stays
 *     within rounding of 2^15.  o is read back as the fp16 value times 2^k: o
 *     rounded to 11 significant bits (bf16 has 8), with no overflow.
 */
lsh_status lsh_chunk_attend(const lsh_config* cfg, const void* qk,
                            const void* v, const int32_t* buckets,
                            const int32_t* perm, void* o_rounds, float* lse,
                            void* stream);

/* Bytes of the o_rounds buffer of lsh_chunk_attend, lsh_chunk_attend_union
 * and lsh_unsort_combine for cfg (0 for an empty or unsupported problem).
 * The caller allocates it; its layout (by cfg->o_format) is given above. */
size_t lsh_o_rounds_bytes(const lsh_config* cfg);

/* Bytes of device workspace lsh_chunk_attend_union needs for cfg (0 for an
 * empty or unsupported problem). */
size_t lsh_union_workspace_bytes(const lsh_config* cfg);

/*
 * lsh_chunk_attend_union -- lsh_chunk_attend with the SET reading of the
 * union over rounds.
 * Follows: Reformer study note, section "Multiple Hash Rounds" (the
 * neighbourhood of token i is the union over r of the per-round
 * neighbourhoods), read as a set: a key found by several rounds counts once.
 *
 *   qk, v, buckets, perm, o_rounds, lse   as for lsh_chunk_attend
 *   inv_perm   [b][H][R][L] int32 (from lsh_sort)
 *   workspace  device scratch of at least lsh_union_workspace_bytes(cfg)
 *              bytes (else LSH_ERR_WORKSPACE_TOO_SMALL); contents ignored
 *
 * As lsh_chunk_attend, except that round r keeps a key j of query i only if
 * j is a key of i in no round before r (a key of i in round r' is one with
 * the same bucket and a sorted slot in the window of i's chunk, under the
 * causal and self rules): every key of the union is attended once, in the
 * first round that finds it, and a round whose keys were all found earlier
 * gives lse = -inf and o = 0.  lsh_unsort_combine of these outputs is then
 * the softmax of s_ij over the set union of the rounds' keys.  Supports
 * n_rounds <= 16 and
 * n_buckets * (seq_len / 64 + 1) < 2^31 (else LSH_ERR_UNSUPPORTED).
 */
lsh_status lsh_chunk_attend_union(const lsh_config* cfg, const void* qk,
                                  const void* v, const int32_t* buckets,
                                  const int32_t* perm, const int32_t* inv_perm,
                                  void* o_rounds, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * lsh_unsort_combine -- back to original order and combine the rounds.
 * Follows: Reformer study note, section "Multiple Hash Rounds" (the
 * neighbourhood of token i is the union over rounds of the per-round
 * neighbourhoods), taken as a multiset: the rounds' softmaxes are merged with
 * weights from their logsumexps.
 *
 *   o_rounds, lse   from lsh_chunk_attend (sorted order; o_rounds in the
 *                   layout described there)
 *   inv_perm        [b][H][R][L] int32 (from lsh_sort)
 *   v               [b][H][L][d] dtype
 *   y               [b][H][L][d] fp32 output, original order
 *
 * y_i = sum_r w_r o_r(i) with w_r = exp(lse_r(i) - M) / sum_r' exp(lse_r'(i) - M),
 * M = max_r lse_r(i), where o_r(i), lse_r(i) are read at slot inv_perm[r][i].
 * If every lse_r(i) is -inf (self-masked token with no other key), y_i = v_i.
 */
lsh_status lsh_unsort_combine(const lsh_config* cfg, const void* o_rounds,
                              const float* lse, const int32_t* inv_perm,
                              const void* v, float* y, void* stream);

/*
 * lsh_local_attend -- local chunked self-attention: the method's attention
 * without hashing.
 * Follows: Reformer overview page "The Reformer - Pushing the limits of
 * language modeling" (yomu.fyi), sections "Approach / What changed" and
 * "Takeaways": the sequence is cut into chunks of length l_c and each chunk
 * also attends to a configurable number of chunks before and after it.
 *
 *   cfg       batch, heads, seq_len, head_dim, chunk_len, causal, self_mask
 *             and dtype as above; n_buckets and n_rounds are not used
 *   n_before  chunks before the query's chunk in its window (>= 0)
 *   n_after   chunks after it (>= 0; no effect when causal)
 *   qk, v     [b][H][L][d]   dtype
 *   y         [b][H][L][d]   fp32 output, original order
 *   lse       [b][H][L]      fp32 output (-inf where no key is left)
 *
 * The keys of query i in chunk c = i / m are the tokens j of chunks
 * max(0, c - n_before) .. min(L/m - 1, c + n_after) with j <= i if causal and
 * j != i if self_mask; with s_ij as for lsh_chunk_attend,
 *   lse_i = log sum_j exp(s_ij),   y_i = sum_j exp(s_ij - lse_i) v_j,
 * and y_i = v_i, lse_i = -inf when there is no key (self-mask only).
 * n_before = 1, n_after = 0 is LSH attention with n_buckets = n_rounds = 1.
 * Windows wider than the sequence are clipped to it.  bf16 inputs use bf16
 * matrix-core products with fp32 accumulation; fp32 inputs use fp32.
 */
lsh_status lsh_local_attend(const lsh_config* cfg, int32_t n_before,
                            int32_t n_after, const void* qk, const void* v,
                            float* y, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * One reversible Reformer layer around the LSH attention.
 * Follows: Reformer study note, sections "Reversible Residual Layers" (the
 * hidden state is split into (x1, x2); y1 = x1 + F(x2), y2 = x2 + G(y1); the
 * inverse x2 = y2 - G(y1), x1 = y1 - F(x2)) and "Chunked Feed-Forward
 * Computation" (G(x) = W2 s(W1 x + b1) + b2 token by token, evaluated over
 * chunks of tokens with the same result).  Here s = ReLU and
 *   F(x) = concat_h(LSHAttn_h(qk_h, v_h)) W_o^T,
 *   qk = bf16(bf16(x) W_qk^T), v = bf16(bf16(x) W_v^T) split into heads of 64
 *   features (head h = features 64h .. 64h+63),
 * with LSHAttn the four calls above (bf16, head_dim = chunk_len = 64).
 * Precision: the inputs of every dense map are rounded to bf16 (nearest,
 * ties to even), products are exact and summed in fp32; qk, v and the hidden
 * activation of G are stored in bf16; the residual stream x1, x2, y1, y2 is
 * fp32 [batch][seq_len][d_model].  Weights are bf16, one row per output
 * feature ([out][in]); biases fp32.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t batch, seq_len;
  int32_t d_model;    /* multiple of 64; heads H = d_model / 64 */
  int32_t d_ff;       /* hidden width of G, multiple of 64 */
  int32_t n_buckets, n_rounds, causal, self_mask;   /* of the LSH attention */
  int32_t ffn_chunk;  /* tokens per chunk of G (0 = all tokens at once) */
} lsh_layer_config;

typedef struct {
  const void* w_qk;   /* [d_model][d_model] bf16 */
  const void* w_v;    /* [d_model][d_model] bf16 */
  const void* w_o;    /* [d_model][d_model] bf16 */
  const void* rot;    /* [H][R][B/2][64] bf16 (may be NULL if B == 1) */
  const void* w_1;    /* [d_ff][d_model] bf16 */
  const float* b_1;   /* [d_ff] */
  const void* w_2;    /* [d_model][d_ff] bf16 */
  const float* b_2;   /* [d_model] */
} lsh_layer_weights;

/*
 * lsh_project_qkv -- the two input maps of F.
 *   x   [b][L][d_model] fp32
 *   qk, v  [b][H][L][64] bf16 outputs (the layout lsh_hash and
 *       lsh_chunk_attend read): qk = bf16(bf16(x) W_qk^T) and likewise v.
 */
lsh_status lsh_project_qkv(const lsh_layer_config* cfg, const float* x,
                           const void* w_qk, const void* w_v, void* qk, void* v,
                           void* stream);

/*
 * lsh_project_out -- the output map of F and its residual add:
 *   out = resid +/- concat_h(bf16(y_att_h)) W_o^T   (minus when subtract = 1)
 *   y_att  [b][H][L][64] fp32 (from lsh_unsort_combine)
 *   resid, out  [b][L][d_model] fp32; out may be the same buffer as resid.
 */
lsh_status lsh_project_out(const lsh_layer_config* cfg, const float* y_att,
                           const void* w_o, const float* resid, int32_t subtract,
                           float* out, void* stream);

/* Bytes of device workspace lsh_ffn needs: one chunk of hidden activations. */
size_t lsh_ffn_workspace_bytes(const lsh_layer_config* cfg);

/*
 * lsh_ffn -- G and its residual add, chunk by chunk of cfg->ffn_chunk tokens:
 *   out = resid +/- (bf16(ReLU(bf16(x) W_1^T + b_1)) W_2^T + b_2)
 *   x, resid, out  [b][L][d_model] fp32; out may be the same buffer as resid
 *   but must not overlap x.  The result does not depend on ffn_chunk.
 */
lsh_status lsh_ffn(const lsh_layer_config* cfg, const float* x, const void* w_1,
                   const float* b_1, const void* w_2, const float* b_2,
                   const float* resid, int32_t subtract, float* out,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace the reversible layer needs (qk, v, the LSH
 * attention's intermediates, the per-head outputs -- kept as bf16, the
 * precision the output map reads them in -- and one FFN chunk). */
size_t lsh_layer_workspace_bytes(const lsh_layer_config* cfg);

/*
 * lsh_reversible_forward -- (y1, y2) = (x1 + F(x2), x2 + G(y1)).
 * lsh_reversible_inverse -- (x1, x2) = (y1 - F(x2), y2 - G(y1)), x2 first.
 * All four tensors [b][L][d_model] fp32; outputs must not overlap inputs.
 * The inverse recomputes F and G from its inputs; it returns the forward's
 * inputs up to the rounding of the fp32 residual adds (and exactly the same
 * F wherever bf16(x2) comes back bit for bit, which then gives the same
 * buckets).
 */
lsh_status lsh_reversible_forward(const lsh_layer_config* cfg,
                                  const lsh_layer_weights* weights,
                                  const float* x1, const float* x2, float* y1,
                                  float* y2, void* workspace,
                                  size_t workspace_bytes, void* stream);
lsh_status lsh_reversible_inverse(const lsh_layer_config* cfg,
                                  const lsh_layer_weights* weights,
                                  const float* y1, const float* y2, float* x1,
                                  float* x2, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* lsh_status_string(lsh_status status);

/* Human-readable detail of the calling thread's last failed call ("" if none). */
const char* lsh_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int lsh_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSH_H_ */
