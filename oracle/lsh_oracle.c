/*
 * lsh_oracle.c -- plain, slow, fp64 CPU oracle of the Reformer LSH-attention
 * forward pass (hash -> sort -> chunked attention -> unsort + round combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the tests, the package smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library: it has its own argument list (plain ints), its
 * own index arithmetic and its own loops.
 *
 * Source of every step ("the pages" = the five web pages on Reformer: The
 * Efficient Transformer, Kitaev, Kaiser, Levskaya, ICLR 2020):
 *   hash      -- Reformer study note (eightmm.github.io), section "LSH
 *                Attention", equation h(x) in {1..B}; the concrete hash is the
 *                random-rotation angular hash argmax([xR ; -xR]).
 *   sort      -- same note, section "Sorting and Chunking" (hash -> sort ->
 *                bucket-contiguous sequence -> chunked attention).
 *   attend    -- same note, "LSH Attention" equations N_LSH(i) and y_i,
 *                "Shared Query-Key Space" (Q = K), "Sorting and Chunking"
 *                (attention inside chunks of nearby sorted positions) and
 *                "Implementation Reading" (causal mask must survive the sort;
 *                same-token policy).
 *   combine   -- same note, "Multiple Hash Rounds", N(i) = union over r of
 *                N^(r)(i), realised as a logsumexp-weighted combine.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - buckets are 0-based indices into the concatenation [xR ; -xR]; ties go
 *     to the lowest index; B = 1 means "no hashing" (bucket 0);
 *   - x.R_j is summed sequentially over k = 0..d-1 in fp64 starting from 0.0;
 *   - the rotation of head h, round r is stored as B/2 direction rows:
 *     rot[h][r][j][k] = R_{h,r}[k][j];
 *   - each (batch, head, round) segment is sorted and chunked independently,
 *     by the key (bucket, original position);
 *   - the window of sorted chunk c is chunk c-1 (if c > 0) and chunk c;
 *   - keys are L2-normalised: k_j = x_j / max(|x_j|_2, 1e-6); score
 *     s_ij = (x_i . k_j) / sqrt(d);
 *   - causal masking compares ORIGINAL positions (j <= i);
 *   - self-mask: token i is never its own candidate in any round; if no round
 *     leaves any candidate, y_i = v_i (the token attends only to itself);
 *   - rounds combine as a multiset: a key found in k rounds counts k times
 *     (oracle_lsh_attend); oracle_lsh_attend_union gives the set reading
 *     instead, where every key of the union counts once: it is attended in
 *     the first round in which it is a candidate and left out of later ones.
 *
 * Layouts (all row-major, all arrays owned by the caller):
 *   qk, v      [batch][heads][L][d]            double
 *   rot        [heads][rounds][B/2][d]         double (empty if B == 1)
 *   buckets    [batch][heads][rounds][L]       int32, original order
 *   perm       [batch][heads][rounds][L]       int32, sorted slot -> position
 *   inv_perm   [batch][heads][rounds][L]       int32, position -> sorted slot
 *   o_rounds   [batch][heads][rounds][L][d]    double, sorted order
 *   lse        [batch][heads][rounds][L]       double, sorted order (-inf = no candidate)
 *   y          [batch][heads][L][d]            double, original order
 *
 * Every function returns 0 on success and -1 on an invalid argument.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_NORM_EPS 1e-6

typedef struct {
  int batch, heads, len, dim, buckets, rounds, chunk, causal, self_mask;
} shape_t;

static int make_shape(shape_t* s, int batch, int heads, int len, int dim,
                      int n_buckets, int rounds, int chunk, int causal,
                      int self_mask) {
  if (batch < 1 || heads < 1 || len < 1 || dim < 1 || rounds < 1 || chunk < 1)
    return -1;
  if (n_buckets < 1 || (n_buckets > 1 && (n_buckets % 2) != 0)) return -1;
  if (len % chunk != 0) return -1;
  s->batch = batch; s->heads = heads; s->len = len; s->dim = dim;
  s->buckets = n_buckets; s->rounds = rounds; s->chunk = chunk;
  s->causal = causal ? 1 : 0; s->self_mask = self_mask ? 1 : 0;
  return 0;
}

/* ------------------------------------------------------------------ hash */

/* Bucket of one token vector x (length d) under one rotation (rows
 * rot_hr[j][k], j < B/2).  The candidates are c = [s_0..s_{B/2-1},
 * -s_0..-s_{B/2-1}] with s_j = sum_k x_k R[k][j]; the bucket is the smallest
 * index t attaining max(c).  s[] is scratch of length B/2. */
static int32_t hash_one(const double* x, const double* rot_hr, int d, int nb,
                        double* s) {
  if (nb == 1) return 0;
  const int half = nb / 2;
  for (int j = 0; j < half; ++j) {
    double acc = 0.0;
    for (int k = 0; k < d; ++k) acc = acc + x[k] * rot_hr[(int64_t)j * d + k];
    s[j] = acc;
  }
  double best = s[0];
  int32_t arg = 0;
  for (int t = 1; t < nb; ++t) {
    const double c = (t < half) ? s[t] : -s[t - half];
    if (c > best) { best = c; arg = t; }
  }
  return arg;
}

/* idx[n] are flat indices into buckets[batch][heads][rounds][L]. */
int oracle_lsh_hash_rows(int batch, int heads, int len, int dim, int n_buckets,
                         int rounds, const double* qk, const double* rot,
                         int64_t n, const int64_t* idx, int32_t* out) {
  shape_t s;
  if (make_shape(&s, batch, heads, len, dim, n_buckets, rounds, len, 0, 0))
    return -1;
  const int64_t total = (int64_t)batch * heads * rounds * len;
  for (int64_t q = 0; q < n; ++q)
    if (idx[q] < 0 || idx[q] >= total) return -1;
  const int half = n_buckets / 2;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double* sbuf = (double*)malloc(sizeof(double) * (size_t)(half > 0 ? half : 1));
    if (!sbuf) bad |= 1;
#pragma omp for schedule(dynamic, 64)
    for (int64_t q = 0; q < n; ++q) {
      if (!sbuf) continue;
      const int64_t f = idx[q];
      const int i = (int)(f % len);
      const int r = (int)((f / len) % rounds);
      const int h = (int)((f / ((int64_t)len * rounds)) % heads);
      const int b = (int)(f / ((int64_t)len * rounds * heads));
      const double* x = qk + (((int64_t)b * heads + h) * len + i) * dim;
      const double* rhr = rot + ((int64_t)h * rounds + r) * half * dim;
      out[q] = hash_one(x, rhr, dim, n_buckets, sbuf);
    }
    free(sbuf);
  }
  return bad ? -1 : 0;
}

int oracle_lsh_hash(int batch, int heads, int len, int dim, int n_buckets,
                    int rounds, const double* qk, const double* rot,
                    int32_t* buckets) {
  const int64_t total = (int64_t)batch * heads * rounds * len;
  if (total <= 0) return -1;
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)total);
  if (!idx) return -1;
  for (int64_t f = 0; f < total; ++f) idx[f] = f;
  const int rc = oracle_lsh_hash_rows(batch, heads, len, dim, n_buckets, rounds,
                                      qk, rot, total, idx, buckets);
  free(idx);
  return rc;
}

/* ------------------------------------------------------------------ sort */

typedef struct { int32_t bucket, pos; } sort_key_t;

static int key_cmp(const void* a, const void* b) {
  const sort_key_t* p = (const sort_key_t*)a;
  const sort_key_t* q = (const sort_key_t*)b;
  if (p->bucket != q->bucket) return p->bucket < q->bucket ? -1 : 1;
  if (p->pos != q->pos) return p->pos < q->pos ? -1 : 1;
  return 0;
}

/* Every (batch, head, round) segment of length L is sorted by the unique key
 * (bucket, original position); perm[s] is the position at sorted slot s and
 * inv_perm is its inverse. */
int oracle_lsh_sort(int n_segments, int len, const int32_t* buckets,
                    int32_t* perm, int32_t* inv_perm) {
  if (n_segments < 1 || len < 1) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int g = 0; g < n_segments; ++g) {
    const int32_t* bk = buckets + (int64_t)g * len;
    sort_key_t* keys = (sort_key_t*)malloc(sizeof(sort_key_t) * (size_t)len);
    if (!keys) { bad |= 1; continue; }
    for (int i = 0; i < len; ++i) { keys[i].bucket = bk[i]; keys[i].pos = i; }
    qsort(keys, (size_t)len, sizeof(sort_key_t), key_cmp);
    for (int s = 0; s < len; ++s) {
      perm[(int64_t)g * len + s] = keys[s].pos;
      inv_perm[(int64_t)g * len + keys[s].pos] = s;
    }
    free(keys);
  }
  return bad ? -1 : 0;
}

/* --------------------------------------------------------------- attend */

/* Candidate keys of the query at sorted slot `slot` of segment `seg`
 * (segment = (b*heads + h)*rounds + r): the original positions j of the
 * tokens in the window of its chunk that share its bucket, satisfy the causal
 * rule and are not the query itself (when self-masking).  Written to out[] in
 * window order; returns their number. */
static int candidates(const shape_t* s, const int32_t* buckets,
                      const int32_t* perm, int64_t seg, int slot,
                      int32_t* out) {
  const int32_t* bk = buckets + seg * s->len;
  const int32_t* pm = perm + seg * s->len;
  const int i = pm[slot];
  const int c = slot / s->chunk;
  const int lo = (c > 0) ? (c - 1) * s->chunk : 0;
  const int hi = (c + 1) * s->chunk;
  int n = 0;
  for (int t = lo; t < hi; ++t) {
    const int j = pm[t];
    if (bk[j] != bk[i]) continue;
    if (s->causal && j > i) continue;
    if (s->self_mask && j == i) continue;
    out[n++] = j;
  }
  return n;
}

static double norm2(const double* x, int d) {
  double acc = 0.0;
  for (int k = 0; k < d; ++k) acc = acc + x[k] * x[k];
  return sqrt(acc);
}

/* 1 when key j is a candidate of query i in some round before round r (the
 * same bucket and, in that round, a sorted slot inside the window of i's
 * chunk; the causal and self rules do not depend on the round, and j already
 * satisfies them as a candidate of round r). */
static int found_earlier(const shape_t* s, const int32_t* buckets,
                         const int32_t* inv_perm, int64_t bh, int r, int i,
                         int j) {
  for (int q = 0; q < r; ++q) {
    const int64_t seg = bh * s->rounds + q;
    const int32_t* bk = buckets + seg * s->len;
    const int32_t* ip = inv_perm + seg * s->len;
    if (bk[i] != bk[j]) continue;
    const int c = ip[i] / s->chunk;
    const int first = (c > 0) ? (c - 1) * s->chunk : 0;
    if (ip[j] >= first && ip[j] < (c + 1) * s->chunk) return 1;
  }
  return 0;
}

/* o (length d) and lse of one query row.  With inv_perm == NULL the rounds
 * are a multiset; otherwise (set semantics of the union over rounds) a key is
 * attended only in the first round in which it is a candidate of the query,
 * so that after the round combine every key of the union weighs once. */
static void attend_one(const shape_t* s, const double* qk, const double* v,
                       const int32_t* buckets, const int32_t* perm,
                       const int32_t* inv_perm, int64_t seg, int slot,
                       int32_t* cand, double* score, double* o, double* lse) {
  const int d = s->dim;
  const int64_t bh = seg / s->rounds;
  const double* xs = qk + bh * (int64_t)s->len * d;
  const double* vs = v + bh * (int64_t)s->len * d;
  const int i = perm[seg * s->len + slot];
  int n = candidates(s, buckets, perm, seg, slot, cand);
  if (inv_perm) {
    const int r = (int)(seg % s->rounds);
    int kept = 0;
    for (int a = 0; a < n; ++a)
      if (!found_earlier(s, buckets, inv_perm, bh, r, i, cand[a])) cand[kept++] = cand[a];
    n = kept;
  }
  for (int k = 0; k < d; ++k) o[k] = 0.0;
  if (n == 0) { *lse = -INFINITY; return; }
  const double* xi = xs + (int64_t)i * d;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  double mx = -INFINITY;
  for (int a = 0; a < n; ++a) {
    const double* xj = xs + (int64_t)cand[a] * d;
    double dot = 0.0;
    for (int k = 0; k < d; ++k) dot = dot + xi[k] * xj[k];
    double nj = norm2(xj, d);
    if (nj < ORACLE_NORM_EPS) nj = ORACLE_NORM_EPS;
    score[a] = dot / nj * inv_sqrt_d;
    if (score[a] > mx) mx = score[a];
  }
  double sum = 0.0;
  for (int a = 0; a < n; ++a) sum += exp(score[a] - mx);
  const double l = mx + log(sum);
  for (int a = 0; a < n; ++a) {
    const double p = exp(score[a] - l);
    const double* vj = vs + (int64_t)cand[a] * d;
    for (int k = 0; k < d; ++k) o[k] += p * vj[k];
  }
  *lse = l;
}

static int attend_rows(int batch, int heads, int len, int dim, int n_buckets,
                       int rounds, int chunk, int causal, int self_mask,
                       const double* qk, const double* v, const int32_t* buckets,
                       const int32_t* perm, const int32_t* inv_perm, int64_t n,
                       const int64_t* idx, double* o, double* lse) {
  shape_t s;
  if (make_shape(&s, batch, heads, len, dim, n_buckets, rounds, chunk, causal,
                 self_mask))
    return -1;
  const int64_t total = (int64_t)batch * heads * rounds * len;
  for (int64_t q = 0; q < n; ++q)
    if (idx[q] < 0 || idx[q] >= total) return -1;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * 2 * (size_t)chunk);
    double* score = (double*)malloc(sizeof(double) * 2 * (size_t)chunk);
    if (!cand || !score) bad |= 1;
#pragma omp for schedule(dynamic, 64)
    for (int64_t q = 0; q < n; ++q) {
      if (!cand || !score) continue;
      attend_one(&s, qk, v, buckets, perm, inv_perm, idx[q] / len,
                 (int)(idx[q] % len), cand, score, o + q * dim, lse + q);
    }
    free(cand);
    free(score);
  }
  return bad ? -1 : 0;
}

/* idx[n] are flat indices seg*L + slot into o_rounds rows / lse. */
int oracle_lsh_attend_rows(int batch, int heads, int len, int dim,
                           int n_buckets, int rounds, int chunk, int causal,
                           int self_mask, const double* qk, const double* v,
                           const int32_t* buckets, const int32_t* perm,
                           int64_t n, const int64_t* idx, double* o,
                           double* lse) {
  return attend_rows(batch, heads, len, dim, n_buckets, rounds, chunk, causal,
                     self_mask, qk, v, buckets, perm, NULL, n, idx, o, lse);
}

int oracle_lsh_attend(int batch, int heads, int len, int dim, int n_buckets,
                      int rounds, int chunk, int causal, int self_mask,
                      const double* qk, const double* v, const int32_t* buckets,
                      const int32_t* perm, double* o_rounds, double* lse) {
  const int64_t total = (int64_t)batch * heads * rounds * len;
  if (total <= 0) return -1;
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)total);
  if (!idx) return -1;
  for (int64_t f = 0; f < total; ++f) idx[f] = f;
  const int rc = oracle_lsh_attend_rows(batch, heads, len, dim, n_buckets,
                                        rounds, chunk, causal, self_mask, qk,
                                        v, buckets, perm, total, idx, o_rounds,
                                        lse);
  free(idx);
  return rc;
}

/* Set semantics of the union over rounds (Reformer study note, "Multiple
 * Hash Rounds": N(i) is the union over r of the per-round neighbourhoods, as
 * a set): per-round o and lse (sorted order, like oracle_lsh_attend) where
 * round r keeps only the candidates that are not candidates of the same query
 * in any round before r, so each key of the union is attended exactly once,
 * in the first round that finds it.  oracle_lsh_combine of these is the
 * softmax over the set union.  inv_perm as returned by oracle_lsh_sort. */
int oracle_lsh_attend_union_rows(int batch, int heads, int len, int dim,
                                 int n_buckets, int rounds, int chunk,
                                 int causal, int self_mask, const double* qk,
                                 const double* v, const int32_t* buckets,
                                 const int32_t* perm, const int32_t* inv_perm,
                                 int64_t n, const int64_t* idx, double* o,
                                 double* lse) {
  if (!inv_perm) return -1;
  return attend_rows(batch, heads, len, dim, n_buckets, rounds, chunk, causal,
                     self_mask, qk, v, buckets, perm, inv_perm, n, idx, o, lse);
}

int oracle_lsh_attend_union(int batch, int heads, int len, int dim,
                            int n_buckets, int rounds, int chunk, int causal,
                            int self_mask, const double* qk, const double* v,
                            const int32_t* buckets, const int32_t* perm,
                            const int32_t* inv_perm, double* o_rounds,
                            double* lse) {
  const int64_t total = (int64_t)batch * heads * rounds * len;
  if (total <= 0) return -1;
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)total);
  if (!idx) return -1;
  for (int64_t f = 0; f < total; ++f) idx[f] = f;
  const int rc = oracle_lsh_attend_union_rows(
      batch, heads, len, dim, n_buckets, rounds, chunk, causal, self_mask, qk, v,
      buckets, perm, inv_perm, total, idx, o_rounds, lse);
  free(idx);
  return rc;
}

/* Candidate list of one query (for tests of the window rule). */
int oracle_lsh_candidates(int batch, int heads, int len, int n_buckets,
                          int rounds, int chunk, int causal, int self_mask,
                          const int32_t* buckets, const int32_t* perm,
                          int64_t seg, int slot, int32_t* out) {
  shape_t s;
  if (make_shape(&s, batch, heads, len, 1, n_buckets, rounds, chunk, causal,
                 self_mask))
    return -1;
  if (seg < 0 || seg >= (int64_t)batch * heads * rounds || slot < 0 ||
      slot >= len)
    return -1;
  return candidates(&s, buckets, perm, seg, slot, out);
}

/* -------------------------------------------------------------- combine */

/* y_i from the R rounds' (o, lse) of token i: softmax weights over the
 * rounds' logsumexps; if every round is empty, y_i = v_i. */
static void combine_one(const shape_t* s, const double* o_rounds,
                        const double* lse, const int32_t* inv_perm,
                        const double* v, int64_t bh, int i, double* y) {
  const int d = s->dim;
  const int64_t L = s->len;
  double mx = -INFINITY;
  for (int r = 0; r < s->rounds; ++r) {
    const int64_t seg = bh * s->rounds + r;
    const double l = lse[seg * L + inv_perm[seg * L + i]];
    if (l > mx) mx = l;
  }
  if (mx == -INFINITY) {
    for (int k = 0; k < d; ++k) y[k] = v[(bh * L + i) * d + k];
    return;
  }
  double wsum = 0.0;
  for (int k = 0; k < d; ++k) y[k] = 0.0;
  for (int r = 0; r < s->rounds; ++r) {
    const int64_t seg = bh * s->rounds + r;
    const int64_t slot = inv_perm[seg * L + i];
    const double w = exp(lse[seg * L + slot] - mx);
    wsum += w;
    for (int k = 0; k < d; ++k) y[k] += w * o_rounds[(seg * L + slot) * d + k];
  }
  for (int k = 0; k < d; ++k) y[k] /= wsum;
}

/* idx[n] are flat indices (b*heads + h)*L + i into y rows. */
int oracle_lsh_combine_rows(int batch, int heads, int len, int dim, int rounds,
                            const double* o_rounds, const double* lse,
                            const int32_t* inv_perm, const double* v,
                            int64_t n, const int64_t* idx, double* y) {
  shape_t s;
  if (make_shape(&s, batch, heads, len, dim, 1, rounds, len, 0, 0)) return -1;
  const int64_t total = (int64_t)batch * heads * len;
  for (int64_t q = 0; q < n; ++q)
    if (idx[q] < 0 || idx[q] >= total) return -1;
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t q = 0; q < n; ++q)
    combine_one(&s, o_rounds, lse, inv_perm, v, idx[q] / len,
                (int)(idx[q] % len), y + q * dim);
  return 0;
}

int oracle_lsh_combine(int batch, int heads, int len, int dim, int rounds,
                       const double* o_rounds, const double* lse,
                       const int32_t* inv_perm, const double* v, double* y) {
  const int64_t total = (int64_t)batch * heads * len;
  if (total <= 0) return -1;
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)total);
  if (!idx) return -1;
  for (int64_t f = 0; f < total; ++f) idx[f] = f;
  const int rc = oracle_lsh_combine_rows(batch, heads, len, dim, rounds,
                                         o_rounds, lse, inv_perm, v, total, idx,
                                         y);
  free(idx);
  return rc;
}

/* -------------------------------------------------------------- forward */

/* All four steps; every intermediate is returned to the caller. */
int oracle_lsh_forward(int batch, int heads, int len, int dim, int n_buckets,
                       int rounds, int chunk, int causal, int self_mask,
                       const double* qk, const double* v, const double* rot,
                       int32_t* buckets, int32_t* perm, int32_t* inv_perm,
                       double* o_rounds, double* lse, double* y) {
  shape_t s;
  if (make_shape(&s, batch, heads, len, dim, n_buckets, rounds, chunk, causal,
                 self_mask))
    return -1;
  if (oracle_lsh_hash(batch, heads, len, dim, n_buckets, rounds, qk, rot,
                      buckets))
    return -1;
  if (oracle_lsh_sort(batch * heads * rounds, len, buckets, perm, inv_perm))
    return -1;
  if (oracle_lsh_attend(batch, heads, len, dim, n_buckets, rounds, chunk,
                        causal, self_mask, qk, v, buckets, perm, o_rounds, lse))
    return -1;
  return oracle_lsh_combine(batch, heads, len, dim, rounds, o_rounds, lse,
                            inv_perm, v, y);
}

/* ------------------------------------------------------- local attention */

/* Local chunked self-attention, the second attention of the method (page 4,
 * "The Reformer - Pushing the limits of language modeling", sections
 * "Approach / What changed" and "Takeaways": the sequence is cut into chunks
 * of length l_c, and each chunk also sees a configurable number of chunks
 * before and after it).  No hashing and no sorting: the candidates of token i
 * in chunk c = i / l_c are the positions of chunks max(0, c - before) ..
 * min(C - 1, c + after), C = L / l_c, filtered by the causal rule (j <= i)
 * and the self-mask (j != i).  Readings where the page is silent: the score,
 * the softmax and the empty-set rule are those of the LSH attention above
 * (Q = K with unit-length keys, 1/sqrt(d), y_i = v_i when no candidate is
 * left), so before = 1, after = 0 is exactly LSH attention with B = 1, R = 1.
 *
 * Layouts: qk, v, y [batch][heads][L][d] double; lse [batch][heads][L]
 * double (-inf = no candidate), all in original order. */
static int local_keeps(const shape_t* s, int i, int j) {
  if (s->causal && j > i) return 0;      /* the future stays hidden */
  if (s->self_mask && j == i) return 0;  /* a token never attends to itself */
  return 1;
}

static void local_one(const shape_t* s, int before, int after,
                      const double* qk, const double* v, int64_t bh, int i,
                      double* score, double* y, double* lse) {
  const int d = s->dim;
  const double* xs = qk + bh * (int64_t)s->len * d;
  const double* vs = v + bh * (int64_t)s->len * d;
  const int nchunks = s->len / s->chunk;
  const int c = i / s->chunk;
  const int c_lo = (c - before > 0) ? c - before : 0;
  const int c_hi = (c + after < nchunks - 1) ? c + after : nchunks - 1;
  const int lo = c_lo * s->chunk;
  const int hi = (c_hi + 1) * s->chunk;
  const double* xi = xs + (int64_t)i * d;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  double mx = -INFINITY;
  int n = 0;
  for (int j = lo; j < hi; ++j) {
    if (!local_keeps(s, i, j)) continue;
    const double* xj = xs + (int64_t)j * d;
    double dot = 0.0;
    for (int k = 0; k < d; ++k) dot = dot + xi[k] * xj[k];
    double nj = norm2(xj, d);
    if (nj < ORACLE_NORM_EPS) nj = ORACLE_NORM_EPS;
    score[j - lo] = dot / nj * inv_sqrt_d;
    if (score[j - lo] > mx) mx = score[j - lo];
    ++n;
  }
  if (n == 0) {
    for (int k = 0; k < d; ++k) y[k] = vs[(int64_t)i * d + k];
    *lse = -INFINITY;
    return;
  }
  double sum = 0.0;
  for (int j = lo; j < hi; ++j)
    if (local_keeps(s, i, j)) sum += exp(score[j - lo] - mx);
  const double lse_i = mx + log(sum);
  for (int k = 0; k < d; ++k) y[k] = 0.0;
  for (int j = lo; j < hi; ++j) {
    if (!local_keeps(s, i, j)) continue;
    const double p = exp(score[j - lo] - lse_i);
    const double* vj = vs + (int64_t)j * d;
    for (int k = 0; k < d; ++k) y[k] += p * vj[k];
  }
  *lse = lse_i;
}

/* idx[n] are flat indices (b*heads + h)*L + i into y rows / lse. */
int oracle_local_attend_rows(int batch, int heads, int len, int dim, int chunk,
                             int before, int after, int causal, int self_mask,
                             const double* qk, const double* v, int64_t n,
                             const int64_t* idx, double* y, double* lse) {
  shape_t s;
  if (make_shape(&s, batch, heads, len, dim, 1, 1, chunk, causal, self_mask))
    return -1;
  if (before < 0 || after < 0) return -1;
  const int64_t total = (int64_t)batch * heads * len;
  for (int64_t q = 0; q < n; ++q)
    if (idx[q] < 0 || idx[q] >= total) return -1;
  /* the window spans at most min(C, before + 1 + after) chunks */
  const int nchunks = len / chunk;
  const int64_t span = (int64_t)before + 1 + after;
  const int64_t wmax = (span < nchunks ? span : nchunks) * (int64_t)chunk;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double* score = (double*)malloc(sizeof(double) * (size_t)wmax);
    if (!score) bad |= 1;
#pragma omp for schedule(dynamic, 64)
    for (int64_t q = 0; q < n; ++q) {
      if (!score) continue;
      local_one(&s, before, after, qk, v, idx[q] / len, (int)(idx[q] % len),
                score, y + q * dim, lse + q);
    }
    free(score);
  }
  return bad ? -1 : 0;
}

int oracle_local_attend(int batch, int heads, int len, int dim, int chunk,
                        int before, int after, int causal, int self_mask,
                        const double* qk, const double* v, double* y,
                        double* lse) {
  const int64_t total = (int64_t)batch * heads * len;
  if (total <= 0) return -1;
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)total);
  if (!idx) return -1;
  for (int64_t f = 0; f < total; ++f) idx[f] = f;
  const int rc = oracle_local_attend_rows(batch, heads, len, dim, chunk, before,
                                          after, causal, self_mask, qk, v,
                                          total, idx, y, lse);
  free(idx);
  return rc;
}

/* ------------------------------------------------------ dense linear maps */

/* out[m][n] = sum_{k=0}^{K-1} a[m][k] * w[n][k] (+ bias[n]), summed in fp64
 * with k ascending from 0.0; w is stored as [N][K] (one row per output
 * feature).  Each output row depends on its own input row only, so any split
 * of the rows into chunks gives the same values (Reformer study note,
 * "Chunked Feed-Forward Computation": the feed-forward map is token-wise). */
int oracle_linear(int64_t rows, int n_out, int n_in, const double* a,
                  const double* w, const double* bias, double* out) {
  if (rows < 0 || n_out < 1 || n_in < 1) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < rows; ++m) {
    const double* am = a + m * (int64_t)n_in;
    for (int n = 0; n < n_out; ++n) {
      const double* wn = w + (int64_t)n * n_in;
      double acc = 0.0;
      for (int k = 0; k < n_in; ++k) acc = acc + am[k] * wn[k];
      out[m * (int64_t)n_out + n] = bias ? acc + bias[n] : acc;
    }
  }
  return 0;
}

/* Thread count of the OpenMP loops above from the next call on (n < 1 leaves
 * it unchanged); returns the count now in force.  Used to time the oracle on
 * one core beside all of them; results do not depend on it. */
int oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
}
