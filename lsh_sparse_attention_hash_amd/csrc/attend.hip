// attend.hip -- attention inside chunks of the bucket-sorted sequence
// (Reformer study note: "LSH Attention" -- same-bucket candidates and the
// softmax-weighted value sum with scores q.k / sqrt(d); "Shared Query-Key
// Space" -- Q = K with unit-length keys; "Sorting and Chunking" -- attention
// over chunks of nearby sorted positions; "Implementation Reading" -- causal
// masking by original position and the same-token policy).
//
// For sorted chunk c of a segment the window is chunks c-1 and c (128 keys);
// the 64 queries are chunk c.  One workgroup (4 waves, 16 queries each) walks
// a run of consecutive chunks: chunk c's rows stay in LDS as chunk c+1's
// predecessor, so each row is gathered from HBM once per round.
//
// bf16: S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 (fp32
// accumulation).  The S^T layout puts one query per lane column, so the
// P^T fragments of two score tiles are directly the B operand of the PV
// product (the contraction over keys is permuted consistently in A and B).
// V is stored transposed in LDS while it is staged.  Each wave skips the
// 16-key tiles of the window in which none of its queries keeps a key (keys
// of other buckets, or past every query under causal masking): in a
// bucket-sorted window most tiles are such, and skipped tiles add only zeros.
// The output rows are
// written as fp32, or (compact format) as fp16 of o * 2^-k with one
// power-of-two scale per (batch, head) taken from the largest |v|
// (vmax_kernel runs first and leaves partial maxima in the header of the
// output buffer; the first workgroup of each head adds k itself to the
// header for the combine; the fp32 accumulation is unchanged).
// fp32: one workgroup per chunk, four threads per query, fp32 arithmetic and
// fp32 output rows.
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "lsh_device.h"
#include "lsh_launch.h"

namespace lsh {

constexpr int kXStride = 72;    // bf16 per x row in LDS (64 + 8 pad: 144 B)
constexpr int kVStride = 136;   // bf16 per V^T row in LDS (128 keys + 8 pad: 272 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNormEps = 1e-6f;

struct AttendArgs {
  const void* qk;
  const void* v;
  const int32_t* buckets;
  const int32_t* perm;
  void* o;               // fp32 rows, or fp16 rows (compact format)
  const float* vpart;    // compact format: partial maxima of |v| per (batch, head)
  int32_t* hexp;         // compact format: scale exponent k per (batch, head)
  float* lse;
  int rounds, L, nchunks, cpw, runs_per_seg, causal, self_mask;
  int64_t blk0;          // fp32 kernel: first block of this launch piece
  // set union over rounds: per-token round keys bucket * (C + 1) + chunk of
  // the token's sorted slot, [b][H][L][ukey_stride] (see union_keys_kernel)
  const int32_t* ukeys;
  int ukey_stride;
};

constexpr int kMaxUnionRounds = 16;
// Set union: the query-side stand-in for rounds a test skips.  (kUnionNoKey -
// w) is 0 or 1 only for w = -4 or -5, and table entries are keys (>= 0) or
// padding (-2).
constexpr int32_t kUnionNoKey = -4;

// ------------------------------------------------------------------- bf16
// V^T rows hold the 128 window keys as 64 dwords (two bf16 keys each) plus 4
// dwords of padding; the dword column is XOR-swizzled by 8 * ((d >> 4) & 3),
// which keeps 4-key groups contiguous and 8-byte aligned while making both the
// transposing writes and the MFMA operand reads free of LDS bank conflicts.
constexpr int kVRowDw = kVStride / 2;   // 68
__device__ __forceinline__ int vt_col(int d, int kdw) { return kdw ^ (8 * ((d >> 4) & 3)); }

struct AttendLds {
  uint16_t xs[128 * kXStride];   // row padding: round keys 0..3 of the set union
  uint32_t vt[kHeadDim * kVRowDw];
  float kinv[128];     // log2(e) / (max(|x_j|, eps) * sqrt(d))
  int32_t kbk[128];    // bucket of the key
  int32_t kpos[128];   // original position of the key
};

// Staging of one sorted chunk (64 rows of x and v), split in two so the
// gathers of the next chunk are in flight while the current one is computed:
// thread t handles the key pair 2*(t/8), 2*(t/8)+1 and the 16-byte column block t%8.
struct ChunkRegs {
  int2 pos;                 // original positions of the two keys
  uint4 xa, xc, va, vc;     // their x and v column blocks
  int ba, bc;               // their bucket ids
  uint4 uk;                 // set union: 4 round keys of key 2*(t/8) + (t%8)/4
};

// The perm entries of this thread's key pair in chunk c, as stored (clamped
// where they are used, so that the load is not waited for here).
__device__ __forceinline__ int2 load_perm_pair(const int32_t* pm, int c) {
  return *reinterpret_cast<const int2*>(pm + (size_t)c * kChunk + 2 * (threadIdx.x >> 3));
}

// Set union: the round keys of rounds 0 .. rnd-1 of the chunk's tokens (at
// the clamped positions pos of this thread's key pair), one 16-byte block of a
// table row per thread.  The load is unconditional (a guarded load would be
// waited for at once): a thread whose block is not needed loads a block of the
// same row, and in round 0 (no earlier round) every thread loads the table's
// first block.  (pos is taken by value: a choice between two fields of the
// register struct would be compiled as a choice of addresses, moving the
// struct to scratch memory.)
template <int UR>
__device__ __forceinline__ uint4 gather_round_keys(int2 pos, const int32_t* uk, int rnd) {
  const int dblk = threadIdx.x & 7;
  const int blk4 = min(4 * (dblk & 3), UR - 4);
  const int tok = (dblk >> 2) ? pos.y : pos.x;
  return load16(uk + (rnd > 0 ? (size_t)tok * UR + blk4 : 0));
}

// The x and v rows, bucket ids and positions of a chunk (and with UKEY its
// round keys for the set union).
template <int UR = 0, bool UKEY = true>
__device__ __forceinline__ void gather_chunk(ChunkRegs& g, int2 pos, int L, const uint16_t* xb,
                                             const uint16_t* vb, const int32_t* bk,
                                             const int32_t* uk = nullptr, int rnd = 0) {
  const int dblk = threadIdx.x & 7;
  pos.x = clamp_index(pos.x, L);
  pos.y = clamp_index(pos.y, L);
  g.pos = pos;
  const size_t ra = (size_t)(pos.x * (kHeadDim / 8) + dblk) * 8;   // elements, < 2^31 * 8
  const size_t rc = (size_t)(pos.y * (kHeadDim / 8) + dblk) * 8;
  g.xa = load16(xb + ra);
  g.xc = load16(xb + rc);
  g.va = load16(vb + ra);
  g.vc = load16(vb + rc);
  g.ba = bk[pos.x];
  g.bc = bk[pos.y];
  if (UR > 0 && UKEY) g.uk = gather_round_keys<UR>(pos, uk, rnd);
}

// Set union: block b (rounds 4b .. 4b+3) of the round keys of window row
// `row`.  Block 0 lives in the 16 padding bytes of the row's x copy, the rest
// in kkey ([128][UR - 4]), which keeps the workgroup's LDS within 40 KB at
// UR = 8 (four workgroups per CU).
template <int UR>
__device__ __forceinline__ int32_t* ukey_block(AttendLds& sm, int32_t* kkey, int row, int b) {
  return b == 0 ? reinterpret_cast<int32_t*>(&sm.xs[row * kXStride + kHeadDim])
                : &kkey[row * (UR - 4) + 4 * (b - 1)];
}

// Write a gathered chunk c into LDS half (c & 1): x rows, V transposed, and
// per-key scale, bucket and position (and the round keys for the set union).
template <int UR = 0>
__device__ __forceinline__ void commit_chunk(AttendLds& sm, const ChunkRegs& g, int c,
                                             int32_t* kkey = nullptr, int rnd = 0) {
  const int tid = threadIdx.x;
  const int p = tid >> 3;          // key pair 0..31
  const int dblk = tid & 7;        // 16-byte column block
  const int row = 64 * (c & 1) + 2 * p;
  if (UR > 0 && 4 * (dblk & 3) < UR && 4 * (dblk & 3) < rnd)
    store16(ukey_block<UR>(sm, kkey, row + (dblk >> 2), dblk & 3), g.uk);
  store16(&sm.xs[row * kXStride + 8 * dblk], g.xa);
  store16(&sm.xs[(row + 1) * kXStride + 8 * dblk], g.xc);
  const uint32_t wa[4] = {g.va.x, g.va.y, g.va.z, g.va.w};
  const uint32_t wc[4] = {g.vc.x, g.vc.y, g.vc.z, g.vc.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t even = (wa[e] & 0xffffu) | (wc[e] << 16);
    const uint32_t odd = (wa[e] >> 16) | (wc[e] & 0xffff0000u);
    const int d0 = 8 * dblk + 2 * e;
    sm.vt[d0 * kVRowDw + vt_col(d0, row >> 1)] = even;
    sm.vt[(d0 + 1) * kVRowDw + vt_col(d0 + 1, row >> 1)] = odd;
  }
  const uint32_t ua[4] = {g.xa.x, g.xa.y, g.xa.z, g.xa.w};
  const uint32_t uc[4] = {g.xc.x, g.xc.y, g.xc.z, g.xc.w};
  float sa = 0.f, sc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = bf16lo(ua[e]), a1 = bf16hi(ua[e]);
    const float c0 = bf16lo(uc[e]), c1 = bf16hi(uc[e]);
    sa += a0 * a0 + a1 * a1;
    sc += c0 * c0 + c1 * c1;
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    sa += __shfl_xor(sa, off);
    sc += __shfl_xor(sc, off);
  }
  if (dblk == 0) {
    // log2(e) / (max(|x|, eps) * sqrt(d)) with sqrt(d) = 8
    sm.kinv[row] = (kLog2e / 8.0f) * __builtin_amdgcn_rsqf(fmaxf(sa, kNormEps * kNormEps));
    sm.kinv[row + 1] = (kLog2e / 8.0f) * __builtin_amdgcn_rsqf(fmaxf(sc, kNormEps * kNormEps));
    sm.kbk[row] = g.ba;
    sm.kbk[row + 1] = g.bc;
    sm.kpos[row] = g.pos.x;
    sm.kpos[row + 1] = g.pos.y;
  }
}

template <bool CAUSAL, bool SELF, int UR, bool O16>
__device__ __forceinline__ void attend_chunk_bf16(AttendLds& sm, const AttendArgs& a, int64_t seg,
                                                  int c, float oscale, int rnd = 0,
                                                  int32_t* kkey = nullptr) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;          // 16-lane group
  const int ql = lane & 15;         // query column of this lane
  const int hq = c & 1, hp = hq ^ 1;
  const int qrow = 64 * hq + 16 * wave + ql;
  const bool first = c == 0;        // chunk 0 has no predecessor (uniform)

  // B operand: Q^T (d x query), lane holds x_q[8*g + 32*ks .. +7]
  bf16x8 qf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) qf[ks] = as_bf16x8(load16(&sm.xs[qrow * kXStride + 8 * g + 32 * ks]));
  const int qb = sm.kbk[qrow];
  const int qp = sm.kpos[qrow];

  // Tiles of the window (16 keys each) that hold no key any query of this
  // wave can keep are skipped: a key whose bucket lies outside the range of
  // the wave's query buckets, or (causal) whose position is past that of every
  // query, is masked for all sixteen.  The bounds are those of queries 0 and 15
  // when they bound all sixteen (bucket-sorted chunks), else they are left open,
  // so the skip never changes a result.
  uint32_t live;   // bit t: window keys 16t .. 16t+15 may hold a kept key
  {
    const int qb0 = __builtin_amdgcn_readfirstlane(qb);
    const int qb15 = __builtin_amdgcn_readlane(qb, 15);
    const bool bsorted = __ballot(qb < qb0 || qb > qb15) == 0;
    const int blo = bsorted ? qb0 : INT_MIN, bhi = bsorted ? qb15 : INT_MAX;
    int phi = INT_MAX;
    if (CAUSAL) {
      const int qp15 = __builtin_amdgcn_readlane(qp, 15);
      if (__ballot(qp > qp15) == 0) phi = qp15;
    }
    const int rp = 64 * hp + lane, rc = 64 * hq + lane;
    const int bkp = sm.kbk[rp], bkc = sm.kbk[rc];
    bool okp = bkp >= blo && bkp <= bhi;
    bool okc = bkc >= blo && bkc <= bhi;
    if (CAUSAL) {
      okp = okp && sm.kpos[rp] <= phi;
      okc = okc && sm.kpos[rc] <= phi;
    }
    const uint64_t mp = first ? 0ull : (uint64_t)__ballot(okp);
    const uint64_t mc = __ballot(okc);
    live = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if ((mp >> (16 * t)) & 0xffffull) live |= 1u << t;
      if ((mc >> (16 * t)) & 0xffffull) live |= 1u << (t + 4);
    }
  }

  // scores, log2-scaled: s[t][i] is key 16t + 4g + i of the window for query ql
  float s[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (!((live >> t) & 1u)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[t][i] = -INFINITY;
      continue;
    }
    const int krow = (16 * t + ql + 64 * hp) & 127;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kf = as_bf16x8(load16(&sm.xs[krow * kXStride + 8 * g + 32 * ks]));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], acc, 0, 0, 0);
    }
    const int row4 = (16 * t + 4 * g + 64 * hp) & 127;
    const float4 kv = *reinterpret_cast<const float4*>(&sm.kinv[row4]);
    const int4 kb = *reinterpret_cast<const int4*>(&sm.kbk[row4]);
    const float kva[4] = {kv.x, kv.y, kv.z, kv.w};
    const int kba[4] = {kb.x, kb.y, kb.z, kb.w};
    int kpa[4] = {0, 0, 0, 0};
    if (CAUSAL || SELF) {
      const int4 kp = *reinterpret_cast<const int4*>(&sm.kpos[row4]);
      kpa[0] = kp.x; kpa[1] = kp.y; kpa[2] = kp.z; kpa[3] = kp.w;
    }
    bool oka[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bool ok = kba[i] == qb;
      if (CAUSAL && SELF) ok = ok && kpa[i] < qp;
      if (CAUSAL && !SELF) ok = ok && kpa[i] <= qp;
      if (!CAUSAL && SELF) ok = ok && kpa[i] != qp;
      oka[i] = ok;
      const float sc = acc[i] * kva[i];
      s[t][i] = ok ? sc : -INFINITY;
    }
    if (UR > 0 && rnd > 0 && __ballot(oka[0] || oka[1] || oka[2] || oka[3])) {
      // each key of the union is attended in the first round that finds it:
      // it is left out here if an earlier round has it as a candidate of this
      // query (same bucket, and its sorted slot in the query's chunk or the
      // one before: round-key difference 0 or 1).  The query's entries for
      // rounds from rnd on are replaced by -4, which lies within 1 of no table
      // entry: keys are >= 0 and padding is -2, while later rounds' keys can be
      // any value below 2^31.  (Any difference is 0 or 1 iff the smallest, as
      // unsigned, is at most 1.)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t dmin = ~0u;
#pragma unroll
        for (int q4 = 0; q4 < UR; q4 += 4) {
          if (q4 < rnd) {
            int4 kq = *reinterpret_cast<const int4*>(ukey_block<UR>(sm, kkey, qrow, q4 / 4));
            if (q4 + 1 >= rnd) kq.y = kUnionNoKey;
            if (q4 + 2 >= rnd) kq.z = kUnionNoKey;
            if (q4 + 3 >= rnd) kq.w = kUnionNoKey;
            const int4 w = *reinterpret_cast<const int4*>(ukey_block<UR>(sm, kkey, row4 + i, q4 / 4));
            dmin = min(min(dmin, (uint32_t)(kq.x - w.x)),
                       min(min((uint32_t)(kq.y - w.y), (uint32_t)(kq.z - w.z)),
                           (uint32_t)(kq.w - w.w)));
          }
        }
        if (dmin <= 1u) s[t][i] = -INFINITY;
      }
    }
  }

  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 8; ++t)
    if ((live >> t) & 1u)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float msafe = (mx == -INFINITY) ? 0.f : mx;

  // probabilities (<= 1) rounded to bf16: the B operand of the PV product
  uint32_t pw[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (!((live >> t) & 1u)) {
      pw[t][0] = pw[t][1] = 0u;
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const bf16x2 pr = {(__bf16)__builtin_amdgcn_exp2f(s[t][i] - msafe),
                         (__bf16)__builtin_amdgcn_exp2f(s[t][i + 1] - msafe)};
      pw[t][i >> 1] = __builtin_bit_cast(uint32_t, pr);
    }
  }

  // O^T = V^T P^T; a fifth tile of ones yields the row sums of the rounded P,
  // so every output row is a weighted mean with weights adding up to one.
  f32x4 oacc[5];
#pragma unroll
  for (int dt = 0; dt < 5; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u,
                                                            0x3f803f80u));
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) {
    if (!((live >> (2 * k2)) & 3u)) continue;
    // MFMA contraction index 8g + j <-> window key 32*k2 + 16*(j/4) + 4g + j%4
    const bf16x8 pb = __builtin_bit_cast(
        bf16x8, make_uint4(pw[2 * k2][0], pw[2 * k2][1], pw[2 * k2 + 1][0], pw[2 * k2 + 1][1]));
    const int c0 = ((32 * k2 + 4 * g + 64 * hp) & 127) >> 1;        // key dword column
    const int c1 = ((32 * k2 + 16 + 4 * g + 64 * hp) & 127) >> 1;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint32_t* vrow = &sm.vt[(16 * dt + ql) * kVRowDw];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (c0 ^ (8 * dt)));
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (c1 ^ (8 * dt)));
      const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, oacc[dt], 0, 0, 0);
    }
    oacc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, oacc[4], 0, 0, 0);
  }

  // the row written as fp32, or as fp16 of o * 2^-k (the power of two oscale
  // folds into the reciprocal exactly)
  const float sum = oacc[4][0];
  const float inv = (sum > 0.f ? __builtin_amdgcn_rcpf(sum) : 0.f) * oscale;
  const int64_t slot = (int64_t)c * kChunk + 16 * wave + ql;
  if (O16) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + ((int64_t)seg * a.L + slot) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const half2v lo = {(_Float16)(oacc[dt][0] * inv), (_Float16)(oacc[dt][1] * inv)};
      const half2v hi = {(_Float16)(oacc[dt][2] * inv), (_Float16)(oacc[dt][3] * inv)};
      *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
  } else {
    float* orow = static_cast<float*>(a.o) + ((int64_t)seg * a.L + slot) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<float4*>(orow + 16 * dt + 4 * g) =
          make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
  }
  if (g == 0)
    a.lse[(int64_t)seg * a.L + slot] =
        (mx == -INFINITY) ? -INFINITY : (mx + __builtin_amdgcn_logf(sum)) * kLn2;
}

// Set union: the rounds of a head differ in cost (round r tests the r rounds
// before it), and under xcd_interleaved_block XCD x works through units x,
// x + 8, x + 16, ...  Rotating each group of 8 units by its group index gives
// XCD x unit (x + g) % 8 of group g, so over 8 groups every XCD takes each
// position in a group (each round, for 8 rounds per head) once.  A bijection
// on [0, units).
__device__ __forceinline__ int64_t rotate_in_group(int64_t unit, int64_t units) {
  if (units % kXcds != 0) return unit;
  const int64_t g = unit / kXcds;
  return g * kXcds + (unit + g) % kXcds;
}

// Four workgroups (waves per SIMD) per CU: at most 128 VGPRs and 40 KB of
// LDS each; the 16-wide round-key table of the set union needs more LDS.
template <bool CAUSAL, bool SELF, int UR, bool O16>
__global__ __launch_bounds__(256, UR > 8 ? 3 : 4) void attend_bf16_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) AttendLds sm;
  __shared__ __attribute__((aligned(16))) int32_t kkey[UR > 4 ? 128 * (UR - 4) : 4];
  const int64_t units = gridDim.x / a.runs_per_seg;
  int64_t blk = xcd_interleaved_block(blockIdx.x, units, a.runs_per_seg);
  if (UR > 0)
    blk = rotate_in_group(blk / a.runs_per_seg, units) * a.runs_per_seg + blk % a.runs_per_seg;
  const int64_t seg = blk / a.runs_per_seg;
  const int run = (int)(blk % a.runs_per_seg);
  const int rnd = UR > 0 ? (int)(seg % a.rounds) : 0;
  const int c0 = run * a.cpw;
  const int c1 = min(a.nchunks, c0 + a.cpw);
  const int64_t bh = seg / a.rounds;
  const uint16_t* xb = static_cast<const uint16_t*>(a.qk) + bh * (int64_t)a.L * kHeadDim;
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + bh * (int64_t)a.L * kHeadDim;
  const int32_t* bk = a.buckets + seg * a.L;
  const int32_t* pm = a.perm + seg * a.L;
  const int32_t* uk = UR > 0 ? a.ukeys + bh * (int64_t)a.L * UR : nullptr;
  // scale of the (batch, head)'s fp16 output rows: 2^-k; the head's first
  // workgroup records k for the combine
  float oscale = 1.0f;
  if (O16) {
    const int k = o_scale_exponent(head_vmax(a.vpart + bh * kVParts));
    oscale = pow2f(-k);
    if (seg % a.rounds == 0 && run == 0 && threadIdx.x == 0) a.hexp[bh] = k;
  }
  ChunkRegs g;
  if (c0 > 0) {
    gather_chunk<UR>(g, load_perm_pair(pm, c0 - 1), a.L, xb, vb, bk, uk, rnd);
    commit_chunk<UR>(sm, g, c0 - 1, kkey, rnd);
  }
  gather_chunk<UR>(g, load_perm_pair(pm, c0), a.L, xb, vb, bk, uk, rnd);
  // perm entries of the chunk after next, requested without a condition (the
  // last chunk's again at the end of the run) so that no wait is forced; in
  // the loop through a descriptor of the run's perm entries, so the address is
  // a scalar base plus this thread's 32-bit offset
  int2 next = load_perm_pair(pm, min(c0 + 1, c1 - 1));
  const __amdgpu_buffer_rsrc_t prun = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(pm + (size_t)c0 * kChunk), (short)0, (c1 - c0) * kChunk * 4, kBufferWord3);
  const int poff = 8 * (threadIdx.x >> 3);
  for (int c = c0; c < c1; ++c) {
    commit_chunk<UR>(sm, g, c, kkey, rnd);
    if (c + 1 < c1) {
      // chunk c+1, in flight during chunk c (its round keys are requested after
      // chunk c: held across it they would push the kernel past 128 VGPRs)
      gather_chunk<UR, false>(g, next, a.L, xb, vb, bk, uk, rnd);
      next = __builtin_bit_cast(int2, __builtin_amdgcn_raw_buffer_load_b64(
                                          prun, poff, (min(c + 2, c1 - 1) - c0) * kChunk * 4, 0));
    }
    __syncthreads();
    attend_chunk_bf16<CAUSAL, SELF, UR, O16>(sm, a, seg, c, oscale, rnd, kkey);
    if (UR > 0 && c + 1 < c1) g.uk = gather_round_keys<UR>(g.pos, uk, rnd);
    __syncthreads();
  }
}

// ------------------------------------------------------------------- fp32
// One workgroup of 256 threads per chunk; the 64 queries are the chunk's
// rows.  The window is taken one 64-key half at a time (the chunk itself,
// then its predecessor): the half's x and v rows are staged in LDS with
// coalesced 16-byte loads, thread t scores query t/4 against keys t%4,
// t%4 + 4, ... of the half, the four threads of a query agree on the running
// maximum, and the half's weights go through LDS so that thread t can sum the
// value features 16*(t%4) .. 16*(t%4)+15 of its query.  fp32 arithmetic, a
// softmax rescaled once between the halves.
constexpr int kF32Row = 68;   // floats per staged row (64 + 4 pad: 4-bank offset per row)

__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  return fmaxf(x, __shfl_xor(x, 2));
}

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  return x + __shfl_xor(x, 2);
}

__global__ __launch_bounds__(256) void attend_f32_kernel(AttendArgs a) {
  __shared__ float xw[kChunk * kF32Row];
  __shared__ float vw[kChunk * kF32Row];
  __shared__ float pw[kChunk * (kChunk + 1)];   // weights [query][key], row padded by 1
  __shared__ float kinv[kChunk];
  __shared__ int32_t kbk[kChunk], kpos[kChunk];
  const int t = threadIdx.x;
  const int qi = t >> 2;      // query of the chunk (scores, outputs)
  const int part = t & 3;     // key residue (scores) / feature block (outputs)
  const int64_t blk = a.blk0 + blockIdx.x;
  const int64_t seg = blk / a.nchunks;
  const int c = (int)(blk % a.nchunks);
  const int64_t bh = seg / a.rounds;
  const float* xb = static_cast<const float*>(a.qk) + bh * (int64_t)a.L * kHeadDim;
  const float* vb = static_cast<const float*>(a.v) + bh * (int64_t)a.L * kHeadDim;
  const int32_t* bk = a.buckets + seg * a.L;
  const int32_t* pm = a.perm + seg * a.L;

  const int qp = clamp_index(pm[(int64_t)c * kChunk + qi], a.L);
  const int qb = bk[qp];
  float4 xq[kHeadDim / 4];
#pragma unroll
  for (int k = 0; k < kHeadDim / 4; ++k)
    xq[k] = *reinterpret_cast<const float4*>(xb + (int64_t)qp * kHeadDim + 4 * k);
  const int32_t* uq = a.ukeys ? a.ukeys + (bh * a.L + qp) * a.ukey_stride : nullptr;
  const int rnd = (int)(seg % a.rounds);   // set union: rounds 0 .. rnd-1 come first

  float m = -INFINITY, l = 0.f;
  float o[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) o[k] = 0.f;

  for (int h = 0; h < (c == 0 ? 1 : 2); ++h) {
    const int cc = c - h;
    // stage: thread t loads columns 16*part .. 16*part+15 of row qi of chunk cc
    const int pos = clamp_index(pm[(int64_t)cc * kChunk + qi], a.L);
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 xv = *reinterpret_cast<const float4*>(xb + (int64_t)pos * kHeadDim + 16 * part + 4 * k);
      const float4 vv = *reinterpret_cast<const float4*>(vb + (int64_t)pos * kHeadDim + 16 * part + 4 * k);
      *reinterpret_cast<float4*>(&xw[qi * kF32Row + 16 * part + 4 * k]) = xv;
      *reinterpret_cast<float4*>(&vw[qi * kF32Row + 16 * part + 4 * k]) = vv;
      ss += xv.x * xv.x + xv.y * xv.y + xv.z * xv.z + xv.w * xv.w;
    }
    ss = quad_sum(ss);
    if (part == 0) {
      kinv[qi] = 1.0f / (fmaxf(sqrtf(ss), kNormEps) * 8.0f);
      kbk[qi] = bk[pos];
      kpos[qi] = pos;
    }
    __syncthreads();

    float sc[16];
    float mh = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = part + 4 * i;
      const float* xr = &xw[kk * kF32Row];
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
      for (int k = 0; k < kHeadDim / 4; ++k) {
        const float4 kv = *reinterpret_cast<const float4*>(xr + 4 * k);
        d0 = fmaf(xq[k].x, kv.x, d0);
        d1 = fmaf(xq[k].y, kv.y, d1);
        d2 = fmaf(xq[k].z, kv.z, d2);
        d3 = fmaf(xq[k].w, kv.w, d3);
      }
      float s = ((d0 + d1) + (d2 + d3)) * kinv[kk];
      const int kp = kpos[kk];
      const bool keep = kbk[kk] == qb && !(a.causal && kp > qp) && !(a.self_mask && kp == qp);
      int seen = 0;
      if (keep && uq) {
        // set union over rounds: the key is attended in the first round that
        // finds it, so it is left out if an earlier round has it as a
        // candidate (round-key difference 0 or 1)
        const int32_t* uj = a.ukeys + (bh * a.L + kp) * a.ukey_stride;
#pragma unroll 1
        for (int r = 0; r < rnd; ++r) seen += (uint32_t)(uq[r] - uj[r]) <= 1u ? 1 : 0;
      }
      if (seen) s = -INFINITY;   // (as a select of the score: a combined condition
                                 // made the compiler move this kernel to scratch)
      sc[i] = keep ? s : -INFINITY;
      mh = fmaxf(mh, sc[i]);
    }
    const float mn = fmaxf(m, quad_max(mh));
    // rescale what the earlier half summed; no key so far leaves it at zero
    const float f = (mn == -INFINITY) ? 0.f : expf(m - mn);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = (mn == -INFINITY) ? 0.f : expf(sc[i] - mn);
      pw[qi * (kChunk + 1) + part + 4 * i] = p;
      ls += p;
    }
    l = l * f + quad_sum(ls);
    m = mn;
    __syncthreads();

    const float* pr = &pw[qi * (kChunk + 1)];
#pragma unroll
    for (int k = 0; k < 16; ++k) o[k] *= f;
    for (int kk = 0; kk < kChunk; ++kk) {
      const float p = pr[kk];
      const float* vr = &vw[kk * kF32Row + 16 * part];
#pragma unroll
      for (int k = 0; k < 16; k += 4) {
        const float4 vv = *reinterpret_cast<const float4*>(vr + k);
        o[k] = fmaf(p, vv.x, o[k]);
        o[k + 1] = fmaf(p, vv.y, o[k + 1]);
        o[k + 2] = fmaf(p, vv.z, o[k + 2]);
        o[k + 3] = fmaf(p, vv.w, o[k + 3]);
      }
    }
    __syncthreads();
  }
  const int64_t slot = (int64_t)c * kChunk + qi;
  float* orow = static_cast<float*>(a.o) + (seg * a.L + slot) * kHeadDim + 16 * part;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int k = 0; k < 16; k += 4)
    *reinterpret_cast<float4*>(orow + k) =
        make_float4(o[k] * inv, o[k + 1] * inv, o[k + 2] * inv, o[k + 3] * inv);
  if (part == 0) a.lse[seg * a.L + slot] = (m == -INFINITY) ? -INFINITY : m + logf(l);
}

// Round r needs the keys of rounds 0 .. r-1 only, so the table holds rounds
// 0 .. R-2, padded to 4, 8 or 16 entries per token.
int union_key_stride(const Shape& s) { return s.rounds <= 5 ? 4 : s.rounds <= 9 ? 8 : kMaxUnionRounds; }

size_t union_workspace_bytes(const Shape& s) {
  return (size_t)s.token_heads() * union_key_stride(s) * sizeof(int32_t);
}

// Round keys of every token for the set union over rounds:
// key_r(t) = bucket_r(t) * (C + 1) + slot_r(t) / m with C = L / m chunks, so
// that key j is a candidate of query i in round r exactly when the two share
// the bucket and j's chunk is i's chunk or the one before, i.e. when
// key_r(i) - key_r(j) is 0 or 1 (C + 1 > C keeps different buckets apart).
template <int RMAX>
__global__ __launch_bounds__(256) void union_keys_kernel(const int32_t* __restrict__ buckets,
                                                        const int32_t* __restrict__ inv_perm,
                                                        int32_t* __restrict__ keys, int rounds,
                                                        int stride, int L, int nb, int64_t total) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= total) return;
  const int64_t bh = g / L;
  const int pos = (int)(g % L);
  const int span = L / kChunk + 1;
  // every round's bucket and slot requested at once (rounds past the last
  // repeat its addresses); padding keys are -2 (the attention masks the
  // rounds a test must skip with kUnionNoKey, -4: no entry lies within 1 of it)
  int32_t bk[RMAX], ip[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int64_t f = (bh * rounds + (r < rounds ? r : rounds - 1)) * L + pos;
    bk[r] = buckets[f];
    ip[r] = inv_perm[f];
  }
  int32_t k[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    k[r] = r < rounds ? min(max(bk[r], 0), nb - 1) * span + clamp_index(ip[r], L) / kChunk : -2;
  int32_t* out = keys + g * stride;
#pragma unroll
  for (int r = 0; r < RMAX; r += 4)
    if (r < stride) *reinterpret_cast<int4*>(out + r) = make_int4(k[r], k[r + 1], k[r + 2], k[r + 3]);
}

// ------------------------------------------------------- fp16 output scale
// Partial maxima of |v| for the scale of the fp16 per-round outputs: part p of
// (batch, head) bh covers rows [p * per, (p + 1) * per), per = ceil(L /
// kVParts).  Finite bf16 magnitudes order like their 15-bit patterns, so the
// maximum is taken on those.  A workgroup takes 256 / TPP consecutive parts,
// TPP threads each (small parts share a workgroup instead of leaving most of
// its threads idle); each thread keeps eight 16-byte pieces in flight.
template <int TPP>
__global__ __launch_bounds__(256) void vmax_kernel(const uint16_t* __restrict__ v,
                                                   float* __restrict__ part, int L,
                                                   int64_t nparts) {
  constexpr int kWaves = 256 / kWave;
  __shared__ uint32_t wmax[kWaves];
  const int64_t gp = (int64_t)blockIdx.x * (256 / TPP) + threadIdx.x / TPP;   // global part
  const int t = threadIdx.x % TPP;
  uint32_t m = 0;
  if (gp < nparts) {
    const int64_t bh = gp / kVParts;
    const int p = (int)(gp % kVParts);
    const int per = (L + kVParts - 1) / kVParts;
    const int r0 = min(L, p * per), r1 = min(L, r0 + per);
    const uint4* src = reinterpret_cast<const uint4*>(v + (bh * L + r0) * kHeadDim);
    const int n = (r1 - r0) * (kHeadDim / 8);   // 16-byte pieces of the part
    for (int i0 = 0; i0 < n; i0 += TPP * 8) {
      uint4 u[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) u[q] = src[min(i0 + TPP * q + t, n - 1)];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t w[4] = {u[q].x & 0x7fff7fffu, u[q].y & 0x7fff7fffu, u[q].z & 0x7fff7fffu,
                               u[q].w & 0x7fff7fffu};
#pragma unroll
        for (int e = 0; e < 4; ++e) m = max(m, max(w[e] & 0xffffu, w[e] >> 16));
      }
    }
  }
  // maximum over the part's TPP threads (lanes of one wave, or whole waves)
#pragma unroll
  for (int off = 1; off < (TPP < kWave ? TPP : kWave); off <<= 1)
    m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if (TPP <= kWave) {
    if (t == 0 && gp < nparts) part[gp] = bf16_to_f32((uint16_t)m);
  } else {
    if (lane_id() == 0) wmax[threadIdx.x / kWave] = m;
    __syncthreads();
    if (t == 0 && gp < nparts) {
      const int w0 = (threadIdx.x / TPP) * (TPP / kWave);
      for (int w = 1; w < TPP / kWave; ++w) m = max(m, wmax[w0 + w]);
      part[gp] = bf16_to_f32((uint16_t)max(m, wmax[w0]));
    }
  }
}

size_t o_header_bytes(const Shape& s) {
  if (!s.o16) return 0;
  // partial maxima [b][H][kVParts] fp32, then exponents [b][H] int32
  const size_t b = (size_t)s.batch * s.heads * (kVParts * sizeof(float) + sizeof(int32_t));
  return (b + 255) & ~(size_t)255;
}

size_t o_rounds_bytes(const Shape& s) {
  return o_header_bytes(s) +
         (size_t)s.segments() * s.len * kHeadDim * (s.o16 ? sizeof(uint16_t) : sizeof(float));
}

template <int UR, bool O16>
static void launch_attend_masks(const AttendArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  if (a.causal && a.self_mask)
    hipLaunchKernelGGL((attend_bf16_kernel<true, true, UR, O16>), grid, block, 0, stream, a);
  else if (a.causal)
    hipLaunchKernelGGL((attend_bf16_kernel<true, false, UR, O16>), grid, block, 0, stream, a);
  else if (a.self_mask)
    hipLaunchKernelGGL((attend_bf16_kernel<false, true, UR, O16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attend_bf16_kernel<false, false, UR, O16>), grid, block, 0, stream, a);
}

template <int UR>
static void launch_attend_stride(const AttendArgs& a, bool o16, dim3 grid, hipStream_t stream) {
  if (o16)
    launch_attend_masks<UR, true>(a, grid, stream);
  else
    launch_attend_masks<UR, false>(a, grid, stream);
}

template <bool UNION>
static hipError_t launch_attend_impl(const Shape& s, const void* qk, const void* v,
                                     const int32_t* buckets, const int32_t* perm,
                                     const int32_t* ukeys, void* o_rounds, float* lse,
                                     hipStream_t stream) {
  AttendArgs a;
  a.ukeys = ukeys;
  a.ukey_stride = UNION ? union_key_stride(s) : 0;
  a.qk = qk;
  a.v = v;
  a.buckets = buckets;
  a.perm = perm;
  a.o = static_cast<char*>(o_rounds) + o_header_bytes(s);
  a.vpart = static_cast<const float*>(o_rounds);
  a.hexp = reinterpret_cast<int32_t*>(static_cast<float*>(o_rounds) +
                                      (int64_t)s.batch * s.heads * kVParts);
  a.lse = lse;
  a.rounds = s.rounds;
  a.L = s.len;
  a.nchunks = s.len / kChunk;
  a.causal = s.causal;
  a.self_mask = s.self_mask;
  const int64_t S = s.segments();
  a.blk0 = 0;
  if (!s.bf16) {
    a.cpw = 1;
    a.runs_per_seg = a.nchunks;
    const int64_t nblk = S * a.nchunks;
    for (int64_t b0 = 0; b0 < nblk; b0 += kMaxBlocks) {
      a.blk0 = b0;
      hipLaunchKernelGGL(attend_f32_kernel, dim3((unsigned)std::min(kMaxBlocks, nblk - b0)),
                         dim3(256), 0, stream, a);
    }
    return hipGetLastError();
  }
  // the scale of the fp16 rows first: partial maxima of |v| into the header
  if (s.o16) {
    const int64_t nparts = (int64_t)s.batch * s.heads * kVParts;
    const int pieces = (s.len + kVParts - 1) / kVParts * (kHeadDim / 8);   // per part
    const uint16_t* vb = static_cast<const uint16_t*>(v);
    float* part = static_cast<float*>(o_rounds);
    // threads per part: about eight pieces each, 32 to 256
    if (pieces <= 32 * 8)
      hipLaunchKernelGGL(vmax_kernel<32>, dim3((unsigned)((nparts + 7) / 8)), dim3(256), 0,
                         stream, vb, part, s.len, nparts);
    else if (pieces <= 64 * 8)
      hipLaunchKernelGGL(vmax_kernel<64>, dim3((unsigned)((nparts + 3) / 4)), dim3(256), 0,
                         stream, vb, part, s.len, nparts);
    else if (pieces <= 128 * 8)
      hipLaunchKernelGGL(vmax_kernel<128>, dim3((unsigned)((nparts + 1) / 2)), dim3(256), 0,
                         stream, vb, part, s.len, nparts);
    else
      hipLaunchKernelGGL(vmax_kernel<256>, dim3((unsigned)nparts), dim3(256), 0, stream, vb,
                         part, s.len, nparts);
  }
  // runs of consecutive chunks per workgroup: long runs re-gather fewer
  // predecessor chunks; keep at least ~2048 workgroups in flight
  const int64_t total = S * a.nchunks;
  int cpw = (int)(total / 2048);
  cpw = cpw < 1 ? 1 : (cpw > 16 ? 16 : cpw);
  a.cpw = cpw;
  a.runs_per_seg = (a.nchunks + cpw - 1) / cpw;
  const dim3 grid((unsigned)(S * a.runs_per_seg));
  if (!UNION)
    launch_attend_stride<0>(a, s.o16, grid, stream);
  else if (a.ukey_stride == 4)
    launch_attend_stride<4>(a, s.o16, grid, stream);
  else if (a.ukey_stride == 8)
    launch_attend_stride<8>(a, s.o16, grid, stream);
  else
    launch_attend_stride<kMaxUnionRounds>(a, s.o16, grid, stream);
  return hipGetLastError();
}

hipError_t launch_attend(const Shape& s, const void* qk, const void* v, const int32_t* buckets,
                         const int32_t* perm, void* o_rounds, float* lse, hipStream_t stream) {
  return launch_attend_impl<false>(s, qk, v, buckets, perm, nullptr, o_rounds, lse, stream);
}

hipError_t launch_attend_union(const Shape& s, const void* qk, const void* v,
                               const int32_t* buckets, const int32_t* perm,
                               const int32_t* inv_perm, void* o_rounds, float* lse,
                               void* workspace, hipStream_t stream) {
  int32_t* keys = static_cast<int32_t*>(workspace);
  const int64_t total = s.token_heads();
  const dim3 kgrid((unsigned)((total + 255) / 256)), kblock(256);
  const int stride = union_key_stride(s);
  if (stride == 4)
    hipLaunchKernelGGL(union_keys_kernel<4>, kgrid, kblock, 0, stream, buckets, inv_perm, keys,
                       s.rounds, stride, s.len, s.buckets, total);
  else if (stride == 8)
    hipLaunchKernelGGL(union_keys_kernel<8>, kgrid, kblock, 0, stream, buckets, inv_perm, keys,
                       s.rounds, stride, s.len, s.buckets, total);
  else
    hipLaunchKernelGGL(union_keys_kernel<kMaxUnionRounds>, kgrid, kblock, 0, stream, buckets,
                       inv_perm, keys, s.rounds, union_key_stride(s), s.len, s.buckets, total);
  return launch_attend_impl<true>(s, qk, v, buckets, perm, keys, o_rounds, lse, stream);
}

}  // namespace lsh
