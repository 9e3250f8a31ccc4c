// hash.hip -- angular LSH bucket ids (Reformer study note, section "LSH
// Attention": a hash h(x) into B buckets; here the random-rotation hash
// bucket = first argmax of [x R ; -x R]) for every token and round.
//
// bf16 inputs: x R is contracted on the matrix cores (v_mfma_f32_32x32x16_bf16,
// exact bf16 products, fp32 accumulation).  The epilogue keeps, per token, the
// two largest |x R_j| as packed keys (magnitude bits with the direction's
// offset in its tile in the low mantissa bits) and the tile of the largest.
// A row is accepted only when the gap between the two best candidates exceeds
// twice a proven bound on the fp32 accumulation error (plus the fp64 rounding
// of the defining sum), so that its bucket is provably the one of the fp64
// definition; the winner's sign then comes from an exact-sign dot product.
// Other rows are listed in LDS and recomputed in fp64, in the defining order,
// by the whole workgroup once its rounds are done.  fp32 inputs are scored in
// fp64 directly.
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
// Rows the fp32 margin cannot certify are settled in fp64 by the whole
// workgroup once its rounds are done: thread t owns directions t, t + 256,
// ... of the row's rotation and loads each as 8 x 16 B.  Each direction's sum
// runs k ascending from 0.0 (the products of two bf16 values are exact, so
// the fused multiply-add rounds exactly like the defining sum).
constexpr int kSettleCap = 1024;   // rows listed per workgroup; the rest are marked in place

__device__ __forceinline__ void settle_take(double s, int j, double& best, int& besti) {
  if (s > best || (s == best && j < besti)) { best = s; besti = j; }
}

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

__device__ __forceinline__ void load_dir(uint4 (&r)[8], const uint16_t* rhr, int j) {
#pragma unroll
  for (int c = 0; c < 8; ++c) r[c] = load16(rhr + (size_t)j * kHeadDim + 8 * c);
}

struct SettleLds {
  double wbest[2][kHashWaves];   // per-wave winners, double-buffered by row parity
  int wbesti[2][kHashWaves];
  float wlow[2][kHashWaves];     // per-wave lower bounds on the best |score|
};

// fp32 score x.R_j (exact bf16 products, fp32 sums) and an upper bound e_j
// on its distance from the definition: the fp32 bound 64 * 2^-22 * 1.01 *
// sum_k |x_k R_kj| of the main loop (the sum itself taken in fp32, with 2^-10
// of slack), plus flush-to-zero slack.
__device__ __forceinline__ void score_fp32(const uint4 (&r)[8], const uint32_t (&xw)[kHeadDim / 2],
                                           float& s, float& ej) {
  float acc = 0.f, aacc = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t w[4] = {r[c].x, r[c].y, r[c].z, r[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xw[4 * c + e]),
                                            __builtin_bit_cast(bf16x2, w[e]), acc, false);
      aacc = __builtin_amdgcn_fdot2_f32_bf16(
          __builtin_bit_cast(bf16x2, xw[4 * c + e] & 0x7fff7fffu),
          __builtin_bit_cast(bf16x2, w[e] & 0x7fff7fffu), aacc, false);
    }
  }
  s = acc;
  ej = aacc * (64.0f * 0x1p-22f * 1.01f * (1.0f + 0x1p-10f)) + 0x1p-117f;
}

// Row e's bucket: the first maximum among the four waves' winners.
__device__ __forceinline__ void settle_pick(const SettleLds& sl, int e, uint32_t ent,
                                            int32_t* out_bh, int tok0, int L) {
  double best = sl.wbest[e & 1][0];
  int besti = sl.wbesti[e & 1][0];
#pragma unroll
  for (int w = 1; w < kHashWaves; ++w) settle_take(sl.wbest[e & 1][w], sl.wbesti[e & 1][w], best, besti);
  out_bh[(size_t)(ent >> 8) * L + tok0 + (int)(ent & 255u)] = besti;
}

// Settles list[0..n): entry (r << 8) | t is token tok0 + t of round r, whose
// x is row t of xsm (bf16, kRowStride apart).  Called by all threads of the
// workgroup; every listed row is written when it returns.
//
// Two passes per row.  The first scores every direction in fp32 with its
// bound e_j, and the workgroup takes the largest lower bound |s_j| - e_j of
// the best |score|.  Only directions whose upper bound |s_j| + e_j reaches
// it can hold the maximum of [xR; -xR] or tie with it; the second pass
// recomputes those in fp64 in the defining order and keeps the first
// maximum.  Each thread remembers its best upper bound (and direction) and
// its second best; when the second best also reaches the lower bound (rare)
// the thread scans its directions again.
// Inlined: as a called function its register saves would raise the kernel's
// register count for the main loop as well.
__device__ __forceinline__ void settle_rows(const uint32_t* list, int n, const uint16_t* xsm,
                                            const uint16_t* rot_h, int32_t* out_bh, int tok0,
                                            int L, int half, SettleLds& sl) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int iters = (half + kHashTokWG - 1) / kHashTokWG;
  const size_t rot_round = (size_t)half * kHeadDim;
  for (int e = 0; e < n; ++e) {
    const uint32_t ent = list[e];
    const int t = (int)(ent & 255u);
    const uint16_t* rhr = rot_h + (size_t)(ent >> 8) * rot_round;
    uint32_t xw[kHeadDim / 2];   // x as packed bf16 pairs
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 u = *reinterpret_cast<const uint4*>(xsm + t * kRowStride + 8 * c);
      xw[4 * c] = u.x;
      xw[4 * c + 1] = u.y;
      xw[4 * c + 2] = u.z;
      xw[4 * c + 3] = u.w;
    }

    // pass 1: fp32 scores; the next direction's row is in flight meanwhile
    float low = -INFINITY, up1 = -INFINITY, up2 = -INFINITY;
    int j1 = -1;
    uint4 rv[8];
    if ((int)threadIdx.x < half) load_dir(rv, rhr, threadIdx.x);
    for (int it = 0; it < iters; ++it) {
      const int j = threadIdx.x + it * kHashTokWG;
      uint4 rn[8];
      const bool next = j + kHashTokWG < half;
      if (next) load_dir(rn, rhr, j + kHashTokWG);
      if (j < half) {
        float sc, ej;
        score_fp32(rv, xw, sc, ej);
        const float up = fabsf(sc) + ej;
        low = fmaxf(low, fabsf(sc) - ej);
        if (up > up1) {
          up2 = up1;
          up1 = up;
          j1 = j;
        } else {
          up2 = fmaxf(up2, up);
        }
      }
      if (next) {
#pragma unroll
        for (int c = 0; c < 8; ++c) rv[c] = rn[c];
      }
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) low = fmaxf(low, __shfl_xor(low, off));
    if (lane == 0) sl.wlow[e & 1][wave] = low;
    __syncthreads();
    if (threadIdx.x == 0 && e > 0) settle_pick(sl, e - 1, list[e - 1], out_bh, tok0, L);
#pragma unroll
    for (int w = 0; w < kHashWaves; ++w) low = fmaxf(low, sl.wlow[e & 1][w]);

    // pass 2: the directions that can reach the maximum, in fp64
    double best = -INFINITY;
    int besti = INT_MAX;
    if (j1 >= 0 && up1 >= low) {
      // opaque to the compiler, so the widened x is not hoisted (64 doubles
      // would not fit beside the main loop's registers)
#pragma unroll
      for (int q = 0; q < kHeadDim / 2; ++q) asm volatile("" : "+v"(xw[q]));
      uint4 r1[8];
      load_dir(r1, rhr, j1);
      const double sd = dot_fp64(r1, xw);
      settle_take(sd, j1, best, besti);
      settle_take(-sd, j1 + half, best, besti);
    }
    if (up2 >= low) {
      for (int it = 0; it < iters; ++it) {
        const int j = threadIdx.x + it * kHashTokWG;
        if (j >= half || j == j1) continue;
        uint4 r2[8];
        load_dir(r2, rhr, j);
        float sc, ej;
        score_fp32(r2, xw, sc, ej);
        if (fabsf(sc) + ej >= low) {
#pragma unroll
          for (int q = 0; q < kHeadDim / 2; ++q) asm volatile("" : "+v"(xw[q]));
          const double sd = dot_fp64(r2, xw);
          settle_take(sd, j, best, besti);
          settle_take(-sd, j + half, best, besti);
        }
      }
    }
    // larger value wins, lower index on equal values: a total order, so any
    // reduction tree finds the first maximum
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const double ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(besti, off);
      settle_take(ob, oi, best, besti);
    }
    if (lane == 0) {
      sl.wbest[e & 1][wave] = best;
      sl.wbesti[e & 1][wave] = besti;
    }
    // the four waves' winners of this row are combined after the next row's
    // first barrier (or the barrier below after the last row)
  }
  __syncthreads();
  if (threadIdx.x == 0 && n > 0) settle_pick(sl, n - 1, list[n - 1], out_bh, tok0, L);
}

// ---------------------------------------------------------------------------
// Keys: the fp32 score with its 5 low mantissa bits replaced by the direction's
// offset inside its 32-direction tile (the lane-half bit 4 of that offset is
// added after the halves merge).  Magnitude keys |key| order like |score| up to
// that truncation; the tile of the running maximum is tracked per lane.
constexpr uint32_t kKeyMask = ~31u;

// Raw buffer descriptor word 3 for gfx9 (32-bit data format; no swizzle): a
// load at a byte offset past the descriptor's size returns zero.
constexpr int kBufferWord3 = 0x00020000;

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

__global__ __launch_bounds__(256) void hash_bf16_kernel(
    const uint16_t* __restrict__ qk, const uint16_t* __restrict__ rot,
    int32_t* __restrict__ buckets, uint32_t* __restrict__ fallback_rows, int heads, int L,
    int half, int rounds) {
  __shared__ __attribute__((aligned(16))) uint16_t rs[2][kStageRows * kRowStride];
  __shared__ float gram_part[kHashWaves];
  __shared__ uint32_t settle_list[kSettleCap];
  __shared__ int settle_n, settle_over;
  __shared__ SettleLds settle_lds;

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  // each XCD takes a contiguous range of (batch, head, token block): its L2
  // then holds the rotations of one or two heads instead of all of them
  const int nblk = (L + kHashTokWG - 1) / kHashTokWG;
  const int64_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int bx = (int)(lb % nblk);
  const size_t bh = (size_t)(lb / nblk);
  const int h = (int)(bh % heads);
  const int tok_wave = bx * kHashTokWG + wave * kHashTokWave;
  const uint16_t* xbase = qk + bh * (size_t)L * kHeadDim;
  const uint16_t* rot_h = rot + (size_t)h * rounds * half * kHeadDim;
  int32_t* out_bh = buckets + bh * rounds * (size_t)L;
  const int tok0 = bx * kHashTokWG;
  if (threadIdx.x == 0) {
    settle_n = 0;
    settle_over = 0;
  }

  // B operand (x^T, k x token): lane holds x[token = lane%32][k = 8*(lane/32) + 16*ks + 0..7].
  // All eight pieces are requested before any is used.  The descriptor covers
  // the wave's tokens below L, so the rows of tokens past L read as zero.
  bf16x8 xf[2][4];
  float xnorm[2];
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
    ss += __shfl_xor(ss, 32);
    xnorm[nb] = sqrtf(ss);
  }

  const int nstages = (half + kStageRows - 1) / kStageRows;
  const int ntiles = (half + 31) / 32;

  for (int r = 0; r < rounds; ++r) {
    const uint16_t* rhr = rot + ((size_t)h * rounds + r) * (size_t)half * kHeadDim;
    float m1[2] = {0.f, 0.f}, m2[2] = {0.f, 0.f};
    int wt[2] = {0, 0};
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
          // Output layout: register i of lane l is direction 32*tile + 8*(i/4) + 4*(l/32) + i%4
          // of token l%32.
          const float before = m1[nb];
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const uint32_t off = 8 * (i >> 2) + (i & 3);
            const uint32_t ka = (__float_as_uint(acc[i]) & kKeyMask) | off;
            const uint32_t kb = (__float_as_uint(acc[i + 1]) & kKeyMask) | (off + 1);
            const float aa = fabsf(__uint_as_float(ka)), ab = fabsf(__uint_as_float(kb));
            const float n1 = fmaxf(m1[nb], fmaxf(aa, ab));
            m2[nb] = fmaxf(m2[nb], __builtin_amdgcn_fmed3f(m1[nb], aa, ab));
            m1[nb] = n1;
          }
          wt[nb] = (__float_as_uint(m1[nb]) != __float_as_uint(before)) ? tile : wt[nb];
        }
      }
      if (more) {
        stage_store(rs[(st + 1) & 1], buf);
        __syncthreads();
      }
    }

    // Largest direction norm of this rotation (all waves' Gram tiles).
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) gmax = fmaxf(gmax, __shfl_xor(gmax, off));
    if (lane == 0) gram_part[wave] = gmax;
    __syncthreads();
    float g2 = gram_part[0];
#pragma unroll
    for (int w = 1; w < kHashWaves; ++w) g2 = fmaxf(g2, gram_part[w]);
    const float rcol = sqrtf(g2 * (1.0f + 0x1p-10f));

    int32_t* bout = buckets + (bh * rounds + r) * (size_t)L;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t own_j = 32u * wt[nb] + (__float_as_uint(m1[nb]) & 31u) + 4u * (lane >> 5);
      const float pm1 = __shfl_xor(m1[nb], 32);
      const float pm2 = __shfl_xor(m2[nb], 32);
      const uint32_t other_j = __shfl_xor(own_j, 32);
      const bool other = pm1 > m1[nb];
      const float w1 = other ? pm1 : m1[nb];
      const float w2 = fmaxf(fminf(m1[nb], pm1), fmaxf(m2[nb], pm2));
      const uint32_t jstar = other ? other_j : own_j;   // the same in lanes l and l^32
      // Sign of the winning score x.R_j*: the two lanes of the token each dot
      // their 32 k-values with the winner's direction row (exact bf16 products,
      // fp32 sums).  On a certified row |x.R_j*| > 2E exceeds the error of any
      // fp32 sum of these 64 products, so the computed sign is exact.
      float part = 0.f;
      {
        const uint16_t* jrow = rhr + (size_t)min(jstar, (uint32_t)(half - 1)) * kHeadDim + 8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint4 rv = load16(jrow + 16 * ks);
          const uint4 xv = __builtin_bit_cast(uint4, xf[nb][ks]);
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.x), __builtin_bit_cast(bf16x2, rv.x), part, false);
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.y), __builtin_bit_cast(bf16x2, rv.y), part, false);
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.z), __builtin_bit_cast(bf16x2, rv.z), part, false);
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xv.w), __builtin_bit_cast(bf16x2, rv.w), part, false);
        }
      }
      const bool pos = part + __shfl_xor(part, 32) > 0.f;
      const float lower1 = __uint_as_float(__float_as_uint(w1) & kKeyMask);
      const float upper2 = __uint_as_float((__float_as_uint(w2) & kKeyMask) + 32u);
      // |fp32 MFMA score - exact| <= 64 * 2^-23 * sum_k |x_k R_kj| <= 64 * 2^-23 |x| |R_j|
      // when each of the 64 additions rounds once, by at most one ulp.  The
      // bound is doubled: the matrix core's internal datapath is not
      // documented, and one that aligns a block of products to its largest
      // exponent and truncates can exceed 64 ulps by a few percent.  The 1%
      // covers the fp64 rounding of the definition; the last terms are
      // flush-to-zero slack.
      const float E = xnorm[nb] * rcol * (64.0f * 0x1p-22f * 1.01f) +
                      (xnorm[nb] + rcol) * 0x1p-120f + 0x1p-118f;
      const bool cert = (lower1 - upper2 > 2.0f * E + lower1 * 0x1p-20f) && (jstar < (uint32_t)half);
      const int bucket = pos ? (int)jstar : (int)jstar + half;

      const int tok = tok_wave + nb * 32 + (lane & 31);
      // rows the fp32 margin cannot certify are listed and settled in fp64
      // later, so no wave waits on them inside the round
      if (lane < 32 && tok < L) {
        if (cert) {
          bout[tok] = bucket;
        } else {
          const int k = atomicAdd(&settle_n, 1);
          if (k < kSettleCap) {
            settle_list[k] = ((uint32_t)r << 8) | (uint32_t)(tok - tok0);
          } else {   // list full: marked in place, found again below
            bout[tok] = -1;
            settle_over = 1;
          }
        }
      }
    }
  }
  __syncthreads();   // the list is complete and the staging buffer is free
  const int n = min(settle_n, kSettleCap);
  if (n == 0) return;
  // the workgroup's x rows (still in registers) into LDS, for the fp64 pass
  uint16_t* xsm = &rs[0][0];   // 256 rows of kRowStride
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      store16(&xsm[(wave * kHashTokWave + nb * 32 + (lane & 31)) * kRowStride + 8 * (lane >> 5) + 16 * ks],
              __builtin_bit_cast(uint4, xf[nb][ks]));
  __syncthreads();
  settle_rows(settle_list, n, xsm, rot_h, out_bh, tok0, L, half, settle_lds);
  uint32_t settled = n;
  if (settle_over) {
    // Only when more than kSettleCap rows of this workgroup were uncertain:
    // collect the rows marked -1 round by round (this workgroup's own
    // writes, visible after the barrier) and settle them.
    for (int r = 0; r < rounds; ++r) {
      if (threadIdx.x == 0) settle_n = 0;
      __syncthreads();
      const int tok = tok0 + threadIdx.x;
      if (tok < L && out_bh[(size_t)r * L + tok] < 0)
        settle_list[atomicAdd(&settle_n, 1)] = ((uint32_t)r << 8) | threadIdx.x;
      __syncthreads();
      const int m = settle_n;
      if (m) settle_rows(settle_list, m, xsm, rot_h, out_bh, tok0, L, half, settle_lds);
      settled += m;
      __syncthreads();   // the list and settle_n are rewritten for the next round
    }
  }
  if (fallback_rows && threadIdx.x == 0 && settled) atomicAdd(fallback_rows, settled);
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
  hipLaunchKernelGGL(hash_bf16_kernel, grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(qk), static_cast<const uint16_t*>(rot), buckets,
                     fallback_rows, s.heads, s.len, half, s.rounds);
  return hipGetLastError();
}

}  // namespace lsh
