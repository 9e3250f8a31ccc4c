// hash.hip -- angular LSH bucket ids (Reformer study note, section "LSH
// Attention": a hash h(x) into B buckets; here the random-rotation hash
// bucket = first argmax of [x R ; -x R]) for every token and round.
//
// bf16 inputs: x R is contracted on the matrix cores (v_mfma_f32_32x32x16_bf16,
// exact bf16 products, fp32 accumulation).  Per token the epilogue tracks the
// largest |x R_j|, its direction, and a bound on every other score, in one of
// two forms (below, chosen by the number of directions).  A row is accepted
// only when the gap between its best score and every other exceeds twice a
// bound on the fp32 accumulation error (plus the fp64 rounding of the
// defining sum), so that its bucket is provably the one of the fp64
// definition; the winner's sign comes from a recomputed dot product.
// Other rows are marked (with a lower bound on their best score) and settled
// by a second kernel, which scores them again with per-direction error bounds
// and recomputes the few directions that can reach the maximum in fp64, in
// the defining order.  fp32 inputs are
// scored in fp64 directly.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "lsh_device.h"
#include "lsh_launch.h"

namespace lsh {

constexpr int kHashWaves = 4;
constexpr int kHashTokWave = 64;                       // two 32-token MFMA column blocks
constexpr int kHashTokWG = kHashWaves * kHashTokWave;  // 256 tokens per workgroup
constexpr int kStageRows = 128;                        // rotation rows staged per LDS pass
constexpr int kRowStride = 72;                         // bf16 per staged row (144 B, padded)

// ---------------------------------------------------------------------------
// Exact bucket of one token, computed by one wave in the defining arithmetic:
// s_j = sum_{k=0..63} x_k R[k][j] in fp64, k ascending from 0.0 (each product
// of two bf16/fp32 values is exact in fp64, so fused or separate multiply-add
// give the same result); candidates +s_j at index j and -s_j at j + half; the
// first (lowest-index) maximum wins.  x: 64 doubles in LDS.
template <typename T>
__device__ __forceinline__ double rot_elem(const T* row, int k);
template <>
__device__ __forceinline__ double rot_elem<uint16_t>(const uint16_t* row, int k) {
  return (double)bf16_to_f32(row[k]);
}
template <>
__device__ __forceinline__ double rot_elem<float>(const float* row, int k) {
  return (double)row[k];
}

template <typename T>
__device__ int exact_bucket(const double* x, const T* rot_hr, int half) {
  const int lane = lane_id();
  double best = -INFINITY;
  int besti = INT_MAX;
  for (int j = lane; j < half; j += kWave) {
    const T* row = rot_hr + (size_t)j * kHeadDim;
    double acc = 0.0;
#pragma unroll 8
    for (int k = 0; k < kHeadDim; ++k) acc = acc + x[k] * rot_elem<T>(row, k);
    // Visit order is not index order (-s_j at j + half comes before +s_{j+64}),
    // so equal values are resolved by index explicitly.
    if (acc > best || (acc == best && j < besti)) { best = acc; besti = j; }
    if (-acc > best || (-acc == best && j + half < besti)) { best = -acc; besti = j + half; }
  }
  // lane-ordered merge: larger value wins, lower index on equal values
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(besti, off);
    if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
  }
  return besti;
}

// ---------------------------------------------------------------------------
// Epilogues.  Register i of a lane holds the score of direction
// 32 t + 8 (i / 4) + 4 (lane / 32) + i % 4 of tile t for token lane % 32; the
// two lanes l and l ^ 32 of a token see disjoint halves of every tile and
// merge after the round.  finish() returns, the same in both lanes of the
// token unless their halves tie (then w1 <= upper2 and the row is not
// certified): the winning direction, a lower bound w1 on its matrix-core
// |score|, an upper bound on the matrix-core |score| of every other direction
// (or, for recomputed ones, on their recomputed value), and the winner's
// recomputed signed value.  A recomputed score (the two lanes of the token
// each dot their 32 k-values with the direction row: exact bf16 products,
// fp32 sums) lies within E of the defining sum, like any fp32 sum of these
// 64 products.
struct Cand {
  uint32_t j;
  float w1, upper2, value;
};

// The recomputed signed scores of N consecutive directions j0 .. j0 + N - 1
// for the token of this lane pair.  Every 16-byte piece of a pair of rows is
// requested before any of them is used.  The descriptor covers the rotation's
// half directions, so rows past half read as zero and score 0, as in the
// padded tile.
template <int N>
__device__ __forceinline__ void recompute(float (&v)[N], __amdgpu_buffer_rsrc_t rrs, uint32_t j0,
                                          const bf16x8 (&x)[4]) {
  const uint32_t lane_off = 16u * (lane_id() >> 5);
#pragma unroll
  for (int e0 = 0; e0 < N; e0 += 2) {
    constexpr int kPair = N < 2 ? N : 2;
    uint4 rv[kPair][4];
#pragma unroll
    for (int e = 0; e < kPair; ++e)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        rv[e][ks] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       rrs, (j0 + e0 + e) * (uint32_t)(kHeadDim * 2) + lane_off + 32u * ks, 0, 0));
    // two rows: keep the scheduler from splitting the requests again (with
    // one row it may move other work in between, which hides their latency)
    if constexpr (N > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < kPair; ++e) {
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 xv = __builtin_bit_cast(uint4, x[ks]);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.x), __builtin_bit_cast(bf16x2, rv[e][ks].x), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.y), __builtin_bit_cast(bf16x2, rv[e][ks].y), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.z), __builtin_bit_cast(bf16x2, rv[e][ks].z), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.w), __builtin_bit_cast(bf16x2, rv[e][ks].w), part, false);
      }
      v[e0 + e] = part + other_half(part);
    }
  }
}

// Keys (fewer directions): every score becomes a key, the fp32 score with its
// 5 low mantissa bits replaced by the direction's offset in the lane's half
// of the tile; the two largest keys are kept (a max3 and a med3 per two
// scores) with the tile of the first.  Magnitude keys order like |score| up
// to that truncation, which the bounds widen by 32 units in the last place.
// Only the winner is recomputed, for its sign.
constexpr uint32_t kKeyMask = ~31u;

struct KeyEpilogue {
  float m1, m2;
  int wt;
  __device__ __forceinline__ void reset() {
    m1 = m2 = 0.f;
    wt = 0;
  }
  __device__ __forceinline__ void tile(const f32x16& acc, int t) {
    const float before = m1;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const uint32_t off = 8 * (i >> 2) + (i & 3);
      const uint32_t ka = (__float_as_uint(acc[i]) & kKeyMask) | off;
      const uint32_t kb = (__float_as_uint(acc[i + 1]) & kKeyMask) | (off + 1);
      const float aa = fabsf(__uint_as_float(ka)), ab = fabsf(__uint_as_float(kb));
      const float n1 = fmaxf(m1, fmaxf(aa, ab));
      m2 = fmaxf(m2, __builtin_amdgcn_fmed3f(m1, aa, ab));
      m1 = n1;
    }
    wt = (__float_as_uint(m1) != __float_as_uint(before)) ? t : wt;
  }
  __device__ __forceinline__ Cand finish(__amdgpu_buffer_rsrc_t rrs, const bf16x8 (&x)[4]) const {
    const uint32_t own_j = 32u * wt + (__float_as_uint(m1) & 31u) + 4u * (lane_id() >> 5);
    const float pm1 = other_half(m1);
    const float pm2 = other_half(m2);
    const uint32_t other_j = other_half(own_j);
    const bool other = pm1 > m1;
    const float w1 = other ? pm1 : m1;
    const float w2 = fmaxf(fminf(m1, pm1), fmaxf(m2, pm2));
    Cand c;
    c.j = other ? other_j : own_j;
    float v[1];
    recompute<1>(v, rrs, c.j, x);
    c.value = v[0];
    c.w1 = __uint_as_float(__float_as_uint(w1) & kKeyMask);
    c.upper2 = __uint_as_float((__float_as_uint(w2) & kKeyMask) + 32u);
    return c;
  }
};

// Quads (many directions): registers 4q .. 4q + 3 form quad q (four
// neighbouring directions).  Per round the epilogue keeps each quad's largest
// |score| over the tiles and the two largest tile maxima with the tile of the
// first: two 3-input maxima per quad and tile, about half the operations of
// the keys per score.  The largest score of the lane lies in the winning quad
// of the winning tile; every other score is bounded by the second tile
// maximum, by the other quads' maxima, or lies in the winning quad, whose
// four scores are recomputed after the round (512 bytes of rows per token and
// round, repaid only when a round has many tiles).
struct QuadEpilogue {
  float pm[4], t1, t2;
  int wt;
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int q = 0; q < 4; ++q) pm[q] = 0.f;
    t1 = t2 = 0.f;
    wt = 0;
  }
  // IEEE-754 maximum (v_maximum3_f32): the scores are finite, and unlike
  // fmaxf it takes the raw matrix-core results without first quieting each
  // one (an extra instruction per score)
  static __device__ __forceinline__ float vmax(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
  }
  __device__ __forceinline__ void tile(const f32x16& acc, int t) {
    float qm[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      qm[q] = vmax(vmax(fabsf(acc[4 * q]), vmax(fabsf(acc[4 * q + 1]), fabsf(acc[4 * q + 2]))),
                   fabsf(acc[4 * q + 3]));
#pragma unroll
    for (int q = 0; q < 4; ++q) pm[q] = vmax(pm[q], qm[q]);
    const float tm = vmax(vmax(qm[0], vmax(qm[1], qm[2])), qm[3]);
    // t1 >= t2 throughout; the first tile reaching the maximum keeps it
    wt = tm > t1 ? t : wt;
    t2 = __builtin_amdgcn_fmed3f(t1, t2, tm);
    t1 = vmax(t1, tm);
  }
  __device__ __forceinline__ Cand finish(__amdgpu_buffer_rsrc_t rrs, const bf16x8 (&x)[4]) const {
    // the quad holding the lane's largest score (first quad on equal values),
    // and the largest of the other quads; s1 == t1
    float s1 = pm[0], s2 = 0.f;
    int qs = 0;
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      qs = pm[q] > s1 ? q : qs;
      s2 = __builtin_amdgcn_fmed3f(s1, s2, pm[q]);
      s1 = fmaxf(s1, pm[q]);
    }
    // u2 bounds every other score of the lane outside the winning quad
    const float u2 = fmaxf(t2, s2);
    const uint32_t own_j = 32u * wt + 8u * qs + 4u * (lane_id() >> 5);
    const float pm1 = other_half(t1);
    const float pu2 = other_half(u2);
    const uint32_t other_j = other_half(own_j);
    const bool other = pm1 > t1;
    const uint32_t j0 = other ? other_j : own_j;
    float v[4];
    recompute<4>(v, rrs, j0, x);
    // The direction with the largest |value| is taken (the first on equal
    // values).  Had the matrix-core maximum been another one of the quad,
    // that one's |value| would be at least w1 - 2E and the row is not
    // certified.
    float vpart = 0.f;
    Cand c;
    c.j = j0;
    c.value = v[0];
#pragma unroll
    for (int e = 1; e < 4; ++e) {
      const bool gt = fabsf(v[e]) > fabsf(c.value);
      vpart = fmaxf(vpart, gt ? fabsf(c.value) : fabsf(v[e]));
      c.j = gt ? j0 + e : c.j;
      c.value = gt ? v[e] : c.value;
    }
    c.w1 = other ? pm1 : t1;
    // the losing half's scores are at most its maximum
    c.upper2 = fmaxf(fmaxf(fminf(t1, pm1), fmaxf(u2, pu2)), vpart);
    return c;
  }
};
// quads for more than this many directions (32 tiles per round)
constexpr int kQuadMinHalf = 1024;

// Stage st of a round: rows [128 st, 128 st + 128) of the rotation, 1024
// pieces of 16 B, 4 per thread.  The descriptor covers only the stage's rows
// below `half`, so the pieces of rows past it read as zero.
__device__ __forceinline__ void stage_load(uint4 (&buf)[4], const uint16_t* rhr, int half,
                                           int st) {
  const int rows = min(kStageRows, half - st * kStageRows);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(rhr + (size_t)st * kStageRows * kHeadDim), (short)0,
      rows * kHeadDim * (int)sizeof(uint16_t), kBufferWord3);
  // piece c = threadIdx.x + 256 q: row c / 8, 16-byte column c % 8
  const uint32_t off = (threadIdx.x >> 3) * (kHeadDim * 2) + (threadIdx.x & 7) * 16;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    buf[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rsrc, off + q * 32 * kHeadDim * 2, 0, 0));
}

__device__ __forceinline__ void stage_store(uint16_t* dst, const uint4 (&buf)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = threadIdx.x + 256 * q;
    store16(&dst[(c >> 3) * kRowStride + (c & 7) * 8], buf[q]);
  }
}

// At most 128 VGPRs (the second bound): four waves per SIMD hide more of the
// matrix-core and LDS latency than three with more registers each.
template <typename Epilogue>
__global__ __launch_bounds__(256, 4) void hash_bf16_kernel(
    const uint16_t* __restrict__ qk, const uint16_t* __restrict__ rot,
    int32_t* __restrict__ buckets, int heads, int L, int half, int rounds) {
  __shared__ __attribute__((aligned(16))) uint16_t rs[2][kStageRows * kRowStride];
  __shared__ float gram_part[kHashWaves];
  // |x| of every token of the workgroup, read once per round for the error
  // bound (held in registers it would push the quad epilogue past 128)
  __shared__ float xnorm_s[2][kHashTokWG];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar
  // each XCD takes a contiguous range of (batch, head, token block): its L2
  // then holds the rotations of one or two heads instead of all of them
  const int nblk = (L + kHashTokWG - 1) / kHashTokWG;
  const int64_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int bx = (int)(lb % nblk);
  const size_t bh = (size_t)(lb / nblk);
  const int h = (int)(bh % heads);
  const int tok_wave = bx * kHashTokWG + wave * kHashTokWave;
  const uint16_t* xbase = qk + bh * (size_t)L * kHeadDim;

  // B operand (x^T, k x token): lane holds x[token = lane%32][k = 8*(lane/32) + 16*ks + 0..7].
  // All eight pieces are requested before any is used.  The descriptor covers
  // the wave's tokens below L, so the rows of tokens past L read as zero.
  bf16x8 xf[2][4];
  {
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(xbase + (size_t)min(tok_wave, L) * kHeadDim), (short)0,
        max(0, min(kHashTokWave, L - tok_wave)) * kHeadDim * (int)sizeof(uint16_t), kBufferWord3);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        xf[nb][ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                        xr, (uint32_t)((nb * 32 + (lane & 31)) * kHeadDim * 2 + (lane >> 5) * 16 + ks * 32),
                        0, 0));
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 u = __builtin_bit_cast(uint4, xf[nb][ks]);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16lo(w[e]), b = bf16hi(w[e]);
        ss += a * a + b * b;
      }
    }
    ss += other_half(ss);
    xnorm_s[nb][threadIdx.x] = sqrtf(ss);   // lanes l and l ^ 32 hold the same value
  }

  const int nstages = (half + kStageRows - 1) / kStageRows;
  const int ntiles = (half + 31) / 32;

  for (int r = 0; r < rounds; ++r) {
    const uint16_t* rhr = rot + ((size_t)h * rounds + r) * (size_t)half * kHeadDim;
    Epilogue ep[2];
    ep[0].reset();
    ep[1].reset();
    float gmax = 0.f;

    uint4 buf[4];
    stage_load(buf, rhr, half, 0);
    __syncthreads();   // previous round's readers of rs[0] are done
    stage_store(rs[0], buf);
    __syncthreads();
    for (int st = 0; st < nstages; ++st) {
      const uint16_t* cur = rs[st & 1];
      const bool more = st + 1 < nstages;
      if (more) stage_load(buf, rhr, half, st + 1);   // in flight during compute

#pragma unroll
      for (int t = 0; t < kStageRows / 32; ++t) {
        const int tile = st * (kStageRows / 32) + t;
        if (tile >= ntiles) break;
        // A operand (R^T, direction x k): lane holds R[k = 8*(lane/32)+16*ks..][j = 32*tile + lane%32].
        bf16x8 a[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          a[ks] = as_bf16x8(load16(&cur[(t * 32 + (lane & 31)) * kRowStride + 8 * (lane >> 5) + 16 * ks]));

        if ((tile & (kHashWaves - 1)) == wave) {
          // The two diagonal 16 x 16 blocks of the Gram matrix R_tile^T R_tile:
          // every direction of the tile lies on one of their diagonals, and an
          // off-diagonal entry never exceeds the larger of its two diagonal
          // ones, so their largest entry is the tile's largest squared
          // direction norm.  Operand of lane l: direction 16 blk + l % 16,
          // k = 32 kh + 8 (l / 16) .. + 7 (the same fragment on both sides).
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
              const bf16x8 r = as_bf16x8(load16(
                  &cur[(t * 32 + blk * 16 + (lane & 15)) * kRowStride + 8 * (lane >> 4) + 32 * kh]));
              g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r, r, g, 0, 0, 0);
            }
            gmax = fmaxf(gmax, fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3])));
          }
        }

#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          f32x16 acc = {};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], xf[nb][ks], acc, 0, 0, 0);
          ep[nb].tile(acc, tile);
        }
      }
      if (more) {
        stage_store(rs[(st + 1) & 1], buf);
        __syncthreads();
      }
    }

    // Largest direction norm of this rotation (all waves' Gram tiles).
    gmax = wave_max(gmax);
    if (lane == 0) gram_part[wave] = gmax;
    __syncthreads();
    float g2 = gram_part[0];
#pragma unroll
    for (int w = 1; w < kHashWaves; ++w) g2 = fmaxf(g2, gram_part[w]);
    const float rcol = sqrtf(g2 * (1.0f + 0x1p-10f));

    int32_t* bout = buckets + (bh * rounds + r) * (size_t)L;
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(uniform_ptr(rhr)), (short)0, half * kHeadDim * (int)sizeof(uint16_t),
        kBufferWord3);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const Cand c = ep[nb].finish(rrs, xf[nb]);
      // |fp32 MFMA score - exact| <= 64 * 2^-23 * sum_k |x_k R_kj| <= 64 * 2^-23 |x| |R_j|
      // when each of the 64 additions rounds once, by at most one ulp.  The
      // bound is doubled: the matrix core's internal datapath is not
      // documented, and one that aligns a block of products to its largest
      // exponent and truncates can exceed 64 ulps by a few percent.  The 1%
      // covers the fp64 rounding of the definition; the last terms are
      // flush-to-zero slack.
      const float xnorm = xnorm_s[nb][threadIdx.x];
      const float E = xnorm * rcol * (64.0f * 0x1p-22f * 1.01f) +
                      (xnorm + rcol) * 0x1p-120f + 0x1p-118f;
      const bool cert = (c.w1 - c.upper2 > 2.0f * E + c.w1 * 0x1p-20f) && (c.j < (uint32_t)half);
      // On a certified row |x.R_j*| > 2E exceeds the error of the recomputed
      // sum, so its sign is exact.
      const int bucket = c.value > 0.f ? (int)c.j : (int)c.j + half;

      const int tok = tok_wave + nb * 32 + (lane & 31);
      // Rows the fp32 margin cannot certify are settled by hash_settle_kernel,
      // so no wave waits on them.  Such a row's entry holds the bitwise
      // complement of a lower bound on its best |x.R_j| (negative: the bound
      // is >= 0): w1 <= |t_j*| <= |s_j*| + E for the defining sum s_j*, less
      // 2^-20 of w1 for the rounding of this subtraction.
      const float lower = fmaxf(c.w1 - E - c.w1 * 0x1p-20f, 0.0f);
      if (lane < 32 && tok < L) bout[tok] = cert ? bucket : (int)~__float_as_uint(lower);
    }
  }
}

// ---------------------------------------------------------------------------
// Settling the rows the main kernel could not certify.  Their entries hold
// ~bits(b) for a lower bound b >= 0 on the row's best |x.R_j| (negative
// values; certified buckets are >= 0).  One workgroup per (segment, range of
// kSettleRange rows) lists the marked rows of its range and settles them
// kSettleBlock at a time against the segment's rotation, so that each
// direction row is read once per block of rows instead of once per row:
//   1. on the matrix cores (v_mfma_f32_16x16x32_bf16: 16 directions x 16
//      rows per product, exact bf16 products and fp32 sums), the score t_j of
//      every direction and A_j = sum_k |x_k| |R_kj| from the products of the
//      absolute values.  e_j = 64 * 2^-22 * 1.01 * (1 + 2^-10) * A_j + 2^-116
//      bounds |t_j - s_j| for the defining fp64 sum s_j: the main loop's
//      bound with sum_k |x_k R_kj| in place of |x| max_j |R_j| (1 + 2^-10
//      covers A_j's own rounding, 2^-116 the flush-to-zero slack of both
//      sums).  Only directions with |t_j| + e_j >= b can hold the maximum of
//      [x R ; -x R] or tie with it; they are listed in LDS;
//   2. the listed directions are recomputed in fp64 in the defining order (k
//      ascending from 0; the products of two bf16 values are exact, so a
//      fused multiply-add rounds like the defining sum), and each row keeps
//      the first maximum (lowest index among equal values): an LDS maximum
//      over the values (nonnegative doubles order like their bit patterns),
//      then an LDS minimum over the indices that reach it.  A block with more
//      candidates than the list holds (rows whose scores all tie, such as
//      all-zero x) is settled by computing every direction in fp64.
// Each wave takes every fourth 16-direction tile, with the next kSettleDepth
// tiles of its share in flight.
constexpr int kSettleRange = 8192;    // rows scanned per workgroup
constexpr int kSettleList = 2048;     // rows listed per pass (more: another pass)
constexpr int kSettleBlock = 16;      // rows settled together (one MFMA column block)
constexpr int kSettleThreads = 256;
constexpr int kSettleDepth = 8;       // tiles in flight per wave
constexpr int kSettleCands = 2048;    // listed candidate (row, direction) pairs per block
constexpr float kSettleErr = 64.0f * 0x1p-22f * 1.01f * (1.0f + 0x1p-10f);

// x . R_j in fp64, k ascending from 0.0 (the defining sum).
__device__ __forceinline__ double dot_fp64(const uint4 (&r)[8], const uint32_t (&xw)[kHeadDim / 2]) {
  double acc = 0.0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t w[4] = {r[c].x, r[c].y, r[c].z, r[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t xv = xw[4 * c + e];
      acc = fma((double)bf16lo(xv), (double)bf16lo(w[e]), acc);
      acc = fma((double)bf16hi(xv), (double)bf16hi(w[e]), acc);
    }
  }
  return acc;
}

// Row `row`'s candidate pair +s_j (index j) and -s_j (index j + half) in
// fp64: the larger value |s_j| as order-preserving bits, offered to the row's
// maximum; returns the index that holds it (j when s_j >= 0).
__device__ __forceinline__ uint64_t settle_value(const uint16_t* rhr, int j, int half,
                                                 const uint16_t* xrow, int& index) {
  uint4 rv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) rv[c] = load16(rhr + (size_t)j * kHeadDim + 8 * c);
  uint32_t xw[kHeadDim / 2];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint4 u = load16(xrow + 8 * c);
    xw[4 * c] = u.x;
    xw[4 * c + 1] = u.y;
    xw[4 * c + 2] = u.z;
    xw[4 * c + 3] = u.w;
  }
  const double sd = dot_fp64(rv, xw);
  index = sd < 0.0 ? j + half : j;
  return (uint64_t)__double_as_longlong(fabs(sd));
}

__device__ __forceinline__ bf16x8 abs_bf16x8(bf16x8 v) {
  uint4 u = __builtin_bit_cast(uint4, v);
  u.x &= 0x7fff7fffu;
  u.y &= 0x7fff7fffu;
  u.z &= 0x7fff7fffu;
  u.w &= 0x7fff7fffu;
  return __builtin_bit_cast(bf16x8, u);
}

// A operand of tile t (directions 16 t .. 16 t + 15): lane l holds
// R[direction 16 t + l % 16][k = 8 (l / 16) + 32 ks .. + 7] for ks = 0, 1.
// Directions past half (and tiles past the last) read as zero.
struct SettleTile {
  bf16x8 a[2];
};

__device__ __forceinline__ void settle_load(SettleTile& tl, __amdgpu_buffer_rsrc_t rsrc, int t) {
  const int lane = lane_id();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    tl.a[ks] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                    rsrc, (uint32_t)((16 * t + (lane & 15)) * kHeadDim * 2 + (lane >> 4) * 16 + ks * 64),
                    0, 0));
}

// acc[i] = t_j, aacc[i] = A_j of direction 16 t + 4 (l / 16) + i and block row l % 16.
__device__ __forceinline__ void settle_scores(const SettleTile& tl, const bf16x8 (&xf)[2],
                                              const bf16x8 (&xa)[2], f32x4& acc, f32x4& aacc) {
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
  aacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl.a[ks], xf[ks], acc, 0, 0, 0);
    aacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abs_bf16x8(tl.a[ks]), xa[ks], aacc, 0, 0, 0);
  }
}

__global__ __launch_bounds__(kSettleThreads, 2) void hash_settle_kernel(
    const uint16_t* __restrict__ qk, const uint16_t* __restrict__ rot,
    int32_t* __restrict__ buckets, uint32_t* __restrict__ fallback_rows, int heads, int L,
    int half, int rounds, int nranges, int64_t blk0) {
  __shared__ int32_t list[kSettleList];
  __shared__ float lbound[kSettleList];            // the listed rows' lower bounds
  __shared__ __attribute__((aligned(16))) uint16_t xs[kSettleBlock * kRowStride];
  __shared__ uint32_t cand[kSettleCands];          // (row << 16) | direction
  __shared__ uint64_t cval[kSettleCands];          // their fp64 values (bits)
  __shared__ int cidx[kSettleCands];               // and the indices holding them
  __shared__ uint64_t rowmax[kSettleBlock];
  __shared__ int rowidx[kSettleBlock];
  __shared__ int nlist, ncand;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  // each XCD takes a contiguous range of (segment, row range): its L2 holds
  // the rotations of few segments
  const int64_t blk = blk0 + xcd_logical_block(blockIdx.x, gridDim.x);
  const int64_t seg = blk / nranges;
  const int range = (int)(blk % nranges);
  const int r = (int)(seg % rounds);
  const int64_t bh = seg / rounds;
  const int h = (int)(bh % heads);
  const int lo = range * kSettleRange;
  const int hi = min(L, lo + kSettleRange);
  int32_t* bk = buckets + seg * L;
  const uint16_t* xb = qk + bh * (size_t)L * kHeadDim;
  const uint16_t* rhr = rot + ((size_t)h * rounds + r) * (size_t)half * kHeadDim;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(rhr), (short)0, half * kHeadDim * (int)sizeof(uint16_t), kBufferWord3);
  const int ntiles = (half + 15) / 16;
  const int nmine = (ntiles - wave + kHashWaves - 1) / kHashWaves;   // tiles wave + 4 q, q < nmine
  const int row = lane & 15;          // the block row this lane scores
  const int dir0 = 4 * (lane >> 4);   // its first direction inside a tile
  uint32_t settled = 0;

  // Passes of at most kSettleList rows: a pass's rows are no longer marked
  // when the next pass scans the range (this workgroup's own writes, ordered
  // by the barriers); a pass that listed every marked row is the last.
  for (;;) {
    if (tid == 0) nlist = 0;
    __syncthreads();
    {  // the marked rows of the range: every load of a thread in flight at once
      constexpr int kPer = kSettleRange / kSettleThreads;
      int32_t v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) v[u] = bk[min(lo + kSettleThreads * u + tid, hi - 1)];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = lo + kSettleThreads * u + tid;
        if (i < hi && v[u] < 0) {
          const int k = atomicAdd(&nlist, 1);
          if (k < kSettleList) {
            list[k] = i;
            lbound[k] = __uint_as_float(~(uint32_t)v[u]);
          }
        }
      }
    }
    __syncthreads();
    const int n = min(nlist, kSettleList);
    const bool more = nlist > kSettleList;   // rows left for another pass
    if (n == 0) break;
    settled += n;

    for (int b0 = 0; b0 < n; b0 += kSettleBlock) {
      const int nrows = min(kSettleBlock, n - b0);
      if (tid < kSettleBlock * 8) {   // the block's x rows into LDS (rows past nrows zero)
        const int rr = tid >> 3, piece = tid & 7;
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (rr < nrows) u = load16(xb + (size_t)list[b0 + rr] * kHeadDim + 8 * piece);
        store16(&xs[rr * kRowStride + 8 * piece], u);
      }
      if (tid < kSettleBlock) {
        rowmax[tid] = 0ull;
        rowidx[tid] = INT_MAX;
      }
      if (tid == 0) ncand = 0;
      __syncthreads();
      // B operand: lane l holds x[row l % 16][k = 8 (l / 16) + 32 ks .. + 7]
      bf16x8 xf[2], xa[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        xf[ks] = as_bf16x8(load16(&xs[row * kRowStride + 8 * (lane >> 4) + 32 * ks]));
        xa[ks] = abs_bf16x8(xf[ks]);
      }
      const bool live = row < nrows;
      const float lowr = lbound[b0 + min(row, nrows - 1)];

      // 1. the directions that can reach the maximum, listed.  Tiles past the
      // wave's share read as zero and fall outside [0, half): steps of
      // kSettleDepth tiles run whole, with no branch between the loads.
      SettleTile ring[kSettleDepth];
#pragma unroll
      for (int d = 0; d < kSettleDepth; ++d) settle_load(ring[d], rsrc, wave + kHashWaves * d);
      for (int q0 = 0; q0 < nmine; q0 += kSettleDepth) {
#pragma unroll
        for (int d = 0; d < kSettleDepth; ++d) {
          const int q = q0 + d;
          f32x4 acc, aacc;
          settle_scores(ring[d], xf, xa, acc, aacc);
          settle_load(ring[d], rsrc, wave + kHashWaves * (q + kSettleDepth));
          const int j0 = 16 * (wave + kHashWaves * q) + dir0;
          uint32_t hit = 0;   // bit i: direction j0 + i can reach the maximum
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = fmaf(aacc[i], kSettleErr, 0x1p-116f);
            hit |= (live && j0 + i < half && fabsf(acc[i]) + e >= lowr) ? 1u << i : 0u;
          }
          if (hit) {   // rare
            const int k = atomicAdd(&ncand, __popc(hit));
            int m = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if ((hit >> i) & 1u) {
                if (k + m < kSettleCands) cand[k + m] = ((uint32_t)row << 16) | (uint32_t)(j0 + i);
                ++m;
              }
            }
          }
        }
      }
      __syncthreads();
      const int nc = ncand;
      // 2. fp64 values; each row's largest, then the lowest index holding it
      if (nc <= kSettleCands) {
        for (int k = tid; k < nc; k += kSettleThreads) {
          const int rr = (int)(cand[k] >> 16), j = (int)(cand[k] & 0xffffu);
          int index;
          const uint64_t v = settle_value(rhr, j, half, &xs[rr * kRowStride], index);
          cval[k] = v;
          cidx[k] = index;
          atomicMax((unsigned long long*)&rowmax[rr], (unsigned long long)v);
        }
        __syncthreads();
        for (int k = tid; k < nc; k += kSettleThreads) {
          const int rr = (int)(cand[k] >> 16);
          if (cval[k] == rowmax[rr]) atomicMin(&rowidx[rr], cidx[k]);
        }
      } else {
        // every direction of every row in fp64 (all scores of some row tie)
        for (int k = tid; k < nrows * half; k += kSettleThreads) {
          const int rr = k / half, j = k % half;
          int index;
          const uint64_t v = settle_value(rhr, j, half, &xs[rr * kRowStride], index);
          atomicMax((unsigned long long*)&rowmax[rr], (unsigned long long)v);
        }
        __syncthreads();
        for (int k = tid; k < nrows * half; k += kSettleThreads) {
          const int rr = k / half, j = k % half;
          int index;
          const uint64_t v = settle_value(rhr, j, half, &xs[rr * kRowStride], index);
          if (v == rowmax[rr]) atomicMin(&rowidx[rr], index);
        }
      }
      __syncthreads();
      if (tid < nrows) bk[list[b0 + tid]] = rowidx[tid];
      __syncthreads();   // xs, the lists and the row tables are rewritten next
    }
    if (!more) break;
  }
  if (fallback_rows && tid == 0 && settled) atomicAdd(fallback_rows, settled);
}

// fp32 inputs: every row in fp64 (one wave per (token, round) row).
__global__ __launch_bounds__(256) void hash_exact_f32_kernel(
    const float* __restrict__ qk, const float* __restrict__ rot, int32_t* __restrict__ buckets,
    int heads, int L, int half, int rounds, int64_t rows, int64_t blk0) {
  __shared__ double xs[4][kHeadDim];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t row = (blk0 + blockIdx.x) * 4 + wave;
  if (row >= rows) return;
  // row indexes buckets[b][H][R][L]
  const int i = (int)(row % L);
  const int64_t seg = row / L;
  const int r = (int)(seg % rounds);
  const int64_t bh = seg / rounds;
  const int h = (int)(bh % heads);
  xs[wave][lane] = (double)qk[(bh * L + i) * kHeadDim + lane];
  __builtin_amdgcn_wave_barrier();
  const int bk = exact_bucket<float>(xs[wave], rot + ((size_t)h * rounds + r) * (size_t)half * kHeadDim,
                                     half);
  if (lane == 0) buckets[row] = bk;
}

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_hash(const Shape& s, const void* qk, const void* rot, int32_t* buckets,
                       uint32_t* fallback_rows, hipStream_t stream) {
  const int64_t rows = s.segments() * s.len;
  if (s.buckets == 1) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       stream, buckets, rows);
    return hipGetLastError();
  }
  const int half = s.buckets / 2;
  if (!s.bf16) {
    const int64_t nblk = (rows + 3) / 4;
    for (int64_t b0 = 0; b0 < nblk; b0 += kMaxBlocks)
      hipLaunchKernelGGL(hash_exact_f32_kernel, dim3((unsigned)std::min(kMaxBlocks, nblk - b0)),
                         dim3(256), 0, stream, static_cast<const float*>(qk),
                         static_cast<const float*>(rot), buckets, s.heads, s.len, half, s.rounds,
                         rows, b0);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((int64_t)(s.len + kHashTokWG - 1) / kHashTokWG * s.heads * s.batch));
  if (half > kQuadMinHalf)
    hipLaunchKernelGGL(hash_bf16_kernel<QuadEpilogue>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(qk), static_cast<const uint16_t*>(rot), buckets,
                       s.heads, s.len, half, s.rounds);
  else
    hipLaunchKernelGGL(hash_bf16_kernel<KeyEpilogue>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(qk), static_cast<const uint16_t*>(rot), buckets,
                       s.heads, s.len, half, s.rounds);
  const int nranges = (s.len + kSettleRange - 1) / kSettleRange;
  const int64_t nblk = s.segments() * nranges;
  for (int64_t b0 = 0; b0 < nblk; b0 += kMaxBlocks)
    hipLaunchKernelGGL(hash_settle_kernel, dim3((unsigned)std::min(kMaxBlocks, nblk - b0)),
                       dim3(kSettleThreads), 0, stream, static_cast<const uint16_t*>(qk),
                       static_cast<const uint16_t*>(rot), buckets, fallback_rows, s.heads, s.len,
                       half, s.rounds, nranges, b0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotations given as d x B/2 matrices ([H][R][d][B/2], rot_cols[h][r][k][j] =
// R_{h,r}[k][j]) rewritten as the direction rows the kernels above read
// ([H][R][B/2][d]).  One workgroup per (matrix, block of 64 directions): the
// 64 x 64 block goes through LDS, read along directions and written along k,
// so both sides are coalesced.  Bits are copied unchanged.
template <typename T>
__global__ __launch_bounds__(256) void rot_rows_kernel(const T* __restrict__ cols,
                                                       T* __restrict__ rows, int half,
                                                       int blocks_per_matrix, int64_t blk0) {
  __shared__ T tile[kHeadDim][kHeadDim + 1];   // [direction][k], padded
  const int64_t blk = blk0 + blockIdx.x;
  const int64_t mat = blk / blocks_per_matrix;
  const int j0 = (int)(blk % blocks_per_matrix) * kHeadDim;
  const T* src = cols + mat * kHeadDim * (int64_t)half;
  T* dst = rows + mat * (int64_t)half * kHeadDim;
  for (int idx = threadIdx.x; idx < kHeadDim * kHeadDim; idx += 256) {
    const int k = idx / kHeadDim, j = idx % kHeadDim;
    if (j0 + j < half) tile[j][k] = src[(int64_t)k * half + j0 + j];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kHeadDim * kHeadDim; idx += 256) {
    const int j = idx / kHeadDim, k = idx % kHeadDim;
    if (j0 + j < half) dst[(int64_t)(j0 + j) * kHeadDim + k] = tile[j][k];
  }
}

hipError_t launch_rot_rows(const Shape& s, const void* rot_cols, void* rot_rows,
                           hipStream_t stream) {
  const int half = s.buckets / 2;
  const int per = (half + kHeadDim - 1) / kHeadDim;
  const int64_t nblk = (int64_t)s.heads * s.rounds * per;
  for (int64_t b0 = 0; b0 < nblk; b0 += kMaxBlocks) {
    const dim3 grid((unsigned)std::min(kMaxBlocks, nblk - b0));
    if (s.bf16)
      hipLaunchKernelGGL(rot_rows_kernel<uint16_t>, grid, dim3(256), 0, stream,
                         static_cast<const uint16_t*>(rot_cols), static_cast<uint16_t*>(rot_rows),
                         half, per, b0);
    else
      hipLaunchKernelGGL(rot_rows_kernel<float>, grid, dim3(256), 0, stream,
                         static_cast<const float*>(rot_cols), static_cast<float*>(rot_rows), half,
                         per, b0);
  }
  return hipGetLastError();
}

}  // namespace lsh
