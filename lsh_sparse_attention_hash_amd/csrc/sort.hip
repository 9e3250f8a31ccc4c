// sort.hip -- stable counting sort of every (batch, head, round) segment by
// bucket id (Reformer study note, section "Sorting and Chunking": tokens are
// sorted by hash bucket so each bucket becomes contiguous).  Because positions
// enter in increasing order and every ranking step keeps that order, the
// result is the order of the unique key (bucket, original position).
//
// B <= 2048: two launches.
//   wide_count    one workgroup per (segment, tile of up to 16,384 keys):
//                 LDS histogram of the tile -> cnt[S][tiles][B]
//   wide_scatter  one workgroup of W waves per (segment, tile): each wave
//                 ranks its share of the tile in position order (per-wave LDS
//                 bucket masks), the workgroup turns the counts into tile-local
//                 bucket starts and global slots (bucket base plus the counts of
//                 the segment's earlier tiles, from cnt), writes inv_perm in
//                 position order and stages the tile's sorted positions in LDS
//                 so that perm leaves in runs of consecutive slots.
// B > 2048: four launches (two for segments of at most 16,384 tokens whose
// tile histograms fit in LDS: prefix, one workgroup per segment, does the
// first three):
//   count    one workgroup per (segment, tile): LDS histogram of the tile
//   scan_t   one thread per (segment, bucket): exclusive prefix over tiles
//   scan_b   one workgroup per segment: exclusive prefix over bucket totals
//   scatter  one workgroup of eight waves per (segment, tile) for B <= 8,192
//            (each wave an eighth of the tile, its offsets from per-wave LDS
//            counts), else one wave per (segment, tile); each wave walks its
//            keys in order, 64 at a time; equal keys inside a batch are
//            ranked by lane through ballots over the key bits, so the
//            scatter is stable.
// Workspace: cnt[S][tiles][B] (B <= 2048); cnt[S][tiles][B] (counts, then
// tile prefixes) and base[S][B] (B > 2048).
#include <algorithm>
#include <mutex>

#include "lsh_device.h"
#include "lsh_launch.h"

namespace lsh {

// Wide tiles (B <= 2048): the tile is the largest of 16,384 ... 1,024 keys
// that still gives at least 256 workgroups (longer tiles write perm in longer
// runs; the workgroups must still cover the chip), with W waves of up to 32
// batches of 64 keys and per-wave bucket tables for up to NB buckets.
constexpr int kWideMaxBuckets = 2048;

struct WidePlan {
  int tile, waves, nbmax, nbat;
};

static WidePlan wide_plan(const Shape& s) {
  WidePlan p;
  p.nbmax = s.buckets <= 256 ? 256 : (s.buckets <= 1024 ? 1024 : 2048);
  const int cap = p.nbmax == 256 ? 4096 : (p.nbmax == 1024 ? 16384 : 8192);
  p.tile = 1024;
  while (p.tile < cap && s.segments() * ((s.len + 2 * p.tile - 1) / (2 * p.tile)) >= 256)
    p.tile *= 2;
  if (p.nbmax == 256)
    p.waves = p.tile >= 4096 ? 8 : 4;
  else if (p.nbmax == 1024)
    p.waves = p.tile >= 8192 ? 8 : 4;
  else
    p.waves = 4;
  p.nbat = p.tile / (kWave * p.waves);
  return p;
}

int sort_tile(const Shape& s) {
  if (s.buckets <= kWideMaxBuckets) return wide_plan(s).tile;
  // at least max(1024, B) keys per tile keeps the count table no larger than
  // the keys; large calls double it up to 4096 while they would have more
  // than 1024 tiles (fewer, longer scatter waves)
  int t = 1024;
  while (t < s.buckets) t <<= 1;
  const int64_t keys = s.segments() * (int64_t)s.len;
  while (t < 4096 && keys / t > 1024) t <<= 1;
  return t;
}

static int64_t sort_tiles(const Shape& s) {
  const int t = sort_tile(s);
  return (s.len + t - 1) / t;
}

size_t sort_workspace_bytes(const Shape& s) {
  const int64_t S = s.segments();
  const int64_t T = sort_tiles(s);
  const size_t cnt = (size_t)S * T * s.buckets * sizeof(int32_t);
  if (s.buckets <= kWideMaxBuckets) return cnt;
  const size_t base = (size_t)S * s.buckets * sizeof(int32_t);
  return ((cnt + 255) & ~(size_t)255) + base;
}

__device__ __forceinline__ int clamp_bucket(int k, int nb) {
  return k < 0 ? 0 : (k >= nb ? nb - 1 : k);
}

constexpr int kCountBatch = 8;

__global__ __launch_bounds__(256) void sort_count_kernel(const int32_t* __restrict__ buckets,
                                                        int32_t* __restrict__ cnt, int L, int nb,
                                                        int tile, int ntiles) {
  extern __shared__ int32_t hist[];
  const int64_t seg = blockIdx.x / ntiles;
  const int t = blockIdx.x % ntiles;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int lo = t * tile;
  const int hi = min(L, lo + tile);
  const int32_t* bk = buckets + seg * L;
  // eight keys per thread requested before any is counted: the loads are
  // unconditional (index clamped to the tile) so that they are all in flight
  for (int i0 = lo; i0 < hi; i0 += 256 * kCountBatch) {
    int32_t k[kCountBatch];
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) k[u] = bk[min(i0 + 256 * u + (int)threadIdx.x, hi - 1)];
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u)
      if (i0 + 256 * u + (int)threadIdx.x < hi) atomicAdd(&hist[clamp_bucket(k[u], nb)], 1);
  }
  __syncthreads();
  int32_t* out = cnt + (seg * ntiles + t) * (int64_t)nb;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) out[i] = hist[i];
}

// cnt[seg][t][bin] -> exclusive prefix over t; totals[seg][bin] = sum over t.
// Loads are issued eight tiles at a time so their latencies overlap.
__global__ __launch_bounds__(256) void sort_scan_tiles_kernel(int32_t* __restrict__ cnt,
                                                             int32_t* __restrict__ totals, int nb,
                                                             int ntiles, int64_t nbins_total,
                                                             int64_t blk0) {
  const int64_t g = (blk0 + blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= nbins_total) return;
  const int64_t seg = g / nb;
  const int bin = (int)(g % nb);
  int32_t* c = cnt + seg * ntiles * (int64_t)nb + bin;
  int32_t run = 0;
  int t = 0;
  for (; t + 8 <= ntiles; t += 8) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c[(int64_t)(t + u) * nb];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c[(int64_t)(t + u) * nb] = run;
      run += v[u];
    }
  }
  for (; t < ntiles; ++t) {
    const int32_t v = c[(int64_t)t * nb];
    c[(int64_t)t * nb] = run;
    run += v;
  }
  totals[g] = run;
}

// totals[seg][bin] -> exclusive prefix over bins (in place).
__global__ __launch_bounds__(1024) void sort_scan_bins_kernel(int32_t* __restrict__ totals,
                                                             int nb) {
  __shared__ int32_t part[1024];
  int32_t* t = totals + (int64_t)blockIdx.x * nb;
  const int per = (nb + 1023) / 1024;
  const int lo = threadIdx.x * per;
  const int hi = min(nb, lo + per);
  int32_t s = 0;
  for (int i = lo; i < hi; ++i) s += t[i];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - s;
  for (int i = lo; i < hi; ++i) {
    const int32_t v = t[i];
    t[i] = run;
    run += v;
  }
}

// One workgroup per segment, for calls whose per-tile histograms fit in LDS:
// count, tile prefixes and bucket bases in one launch.  Every tile's
// histogram is built in LDS from the segment's keys (sixteen loads per thread
// in flight), each thread then walks its bins over the tiles, writing the
// exclusive prefixes the scatter reads, and a block scan over the bin totals
// gives the bucket bases.  Same outputs as count + scan_t + scan_b.
constexpr int kPrefixThreads = 1024;
constexpr int kPrefixLdsInts = 32768;   // 128 KB of histograms
constexpr int kPrefixMaxLen = 16384;    // longest segment counted by one workgroup

__global__ __launch_bounds__(kPrefixThreads) void sort_prefix_kernel(
    const int32_t* __restrict__ buckets, int32_t* __restrict__ cnt, int32_t* __restrict__ base,
    int L, int nb, int tile, int ntiles) {
  __shared__ int32_t hist[kPrefixLdsInts];
  __shared__ int32_t part[kPrefixThreads];
  const int tid = threadIdx.x;
  const int64_t seg = blockIdx.x;
  const int cells = ntiles * nb;
  for (int i = tid; i < cells; i += kPrefixThreads) hist[i] = 0;
  __syncthreads();
  const int32_t* bk = buckets + seg * L;
  for (int i0 = 0; i0 < L; i0 += kPrefixThreads * 16) {
    int32_t k[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) k[u] = bk[min(i0 + kPrefixThreads * u + tid, L - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + kPrefixThreads * u + tid;
      if (i < L) atomicAdd(&hist[(i / tile) * nb + clamp_bucket(k[u], nb)], 1);
    }
  }
  __syncthreads();
  // bins tid*per .. tid*per+per-1: exclusive prefixes over the tiles
  const int per = (nb + kPrefixThreads - 1) / kPrefixThreads;
  int32_t* out = cnt + seg * (int64_t)ntiles * nb;
  int32_t mine = 0;
  for (int q = 0; q < per; ++q) {
    const int b = tid * per + q;
    if (b >= nb) break;
    int32_t run = 0;
    for (int t = 0; t < ntiles; ++t) {
      const int32_t c = hist[t * nb + b];
      out[(int64_t)t * nb + b] = run;
      run += c;
    }
    hist[b] = run;   // tile 0's counts are no longer needed: bin totals
    mine += run;
  }
  part[tid] = mine;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums
  for (int off = 1; off < kPrefixThreads; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t acc = part[tid] - mine;
  int32_t* bs = base + seg * nb;
  for (int q = 0; q < per; ++q) {
    const int b = tid * per + q;
    if (b >= nb) break;
    bs[b] = acc;
    acc += hist[b];
  }
}

// One wave per (segment, tile) (B > 2048).  The tile's keys are first loaded
// into registers (kScatterBatches loads in flight per lane), then ranked 64 at
// a time in position order; each key's slot is its bucket's running offset
// (LDS) plus its rank among the equal keys of lower lanes, found by
// intersecting the ballots of every key bit.
constexpr int kScatterBatches = 32;   // keys taken 32 batches of 64 at a time

__global__ __launch_bounds__(64) void sort_scatter_kernel(
    const int32_t* __restrict__ buckets, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ base, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int L, int nb, int nbits, int tile, int ntiles) {
  extern __shared__ int32_t run[];   // [nb] running slot of each bucket
  const int lane = lane_id();
  // each XCD scatters whole segments, so a segment's perm lines fill up in one
  // L2 before they are written back
  const int64_t blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int64_t seg = blk / ntiles;
  const int t = (int)(blk % ntiles);
  const int32_t* pre = cnt + (seg * ntiles + t) * (int64_t)nb;
  const int32_t* bs = base + seg * nb;
  const int lo = t * tile;
  const int hi = min(L, lo + tile);
  const int32_t* bk = buckets + seg * L;
  int32_t* pm = perm + seg * L;
  int32_t* ip = inv_perm + seg * L;

  // bucket offsets of this tile, sixteen per lane requested at once
  for (int i0 = 0; i0 < nb; i0 += kWave * 16) {
    int32_t bv[16], pv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = min(i0 + kWave * u + lane, nb - 1);
      bv[u] = bs[i];
      pv[u] = pre[i];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + kWave * u + lane;
      if (i < nb) run[i] = bv[u] + pv[u];
    }
  }
  __builtin_amdgcn_wave_barrier();

  for (int c0 = lo; c0 < hi; c0 += kWave * kScatterBatches) {
    // unconditional loads (index clamped to the tile), so all are in flight
    int key[kScatterBatches];
#pragma unroll
    for (int b = 0; b < kScatterBatches; ++b) key[b] = bk[min(c0 + b * kWave + lane, hi - 1)];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int b = 0; b < kScatterBatches; ++b) {
      const int i0 = c0 + b * kWave;
      if (i0 >= hi) break;
      const int i = i0 + lane;
      const bool valid = i < hi;
      const int k = valid ? clamp_bucket(key[b], nb) : 0;
      uint64_t peers = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (k >> bit) & 1;
        const uint64_t ones = __ballot(set);
        peers &= set ? ones : ~ones;
      }
      const int32_t start = valid ? run[k] : 0;
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
      const int n = __popcll(peers);
      __builtin_amdgcn_wave_barrier();
      if (valid && rank == n - 1) run[k] = start + n;
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        const int32_t slot = start + rank;
        pm[slot] = i;
        ip[i] = slot;
      }
    }
  }
}

// The same with the tile split over eight waves (B <= 8,192), so that a
// tile's keys are ranked by eight waves at once.  Each wave takes an eighth
// of the tile in position order.  Pass 1 counts every wave's keys per bucket
// (LDS atomics on 16-bit halves of 32-bit words: an eighth of a tile holds
// at most 1,024 keys); the counts then become each wave's offset inside the
// tile's run of every bucket (the counts of the waves before it); pass 2
// ranks the keys 64 at a time like the one-wave form, each key's slot being
// its bucket's first slot in the tile plus its wave's running offset plus
// its rank among the equal keys of lower lanes.  The tables take all 160 KB
// of the CU's LDS at B = 8,192 (one workgroup per CU); against one wave per
// tile the scatter at 4 x 524,288 tokens and 8,192 buckets takes 83 instead
// of 128 us (four waves: 102 us).
constexpr int kSplitMaxBuckets = 8192;
constexpr int kSplitWaves = 8;

// `totals`: every bucket's count in the segment ([S][B], from scan_t).
__global__ __launch_bounds__(kWave * kSplitWaves) void sort_scatter_split_kernel(
    const int32_t* __restrict__ buckets, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ totals, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int L, int nb, int nbits, int tile, int ntiles) {
  __shared__ int32_t run[kSplitMaxBuckets];                       // the tile's first slot
  __shared__ uint32_t hw[kSplitWaves * kSplitMaxBuckets / 2];     // 16-bit per (wave, bucket)
  constexpr int kThreads = kWave * kSplitWaves;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid >> 6;
  const int64_t blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int64_t seg = blk / ntiles;
  const int t = (int)(blk % ntiles);
  const int32_t* pre = cnt + (seg * ntiles + t) * (int64_t)nb;
  const int32_t* bs = totals + seg * nb;
  const int lo = t * tile;
  const int hi = min(L, lo + tile);
  const int sub = tile / kSplitWaves;   // a multiple of 64 (tiles here hold >= 4,096 keys)
  const int wlo = min(hi, lo + w * sub);
  const int whi = min(hi, wlo + sub);
  const int32_t* bk = buckets + seg * L;
  int32_t* pm = perm + seg * L;
  int32_t* ip = inv_perm + seg * L;
  uint16_t* h16 = reinterpret_cast<uint16_t*>(hw) + w * nb;   // this wave's table

  // The tile's first slot of every bucket: the bucket's base in the segment
  // (the exclusive prefix over buckets of the segment's totals, computed here
  // by every workgroup of the segment) plus the counts of the segment's
  // earlier tiles.  Thread tid takes buckets 16 tid .. 16 tid + 15; the
  // waves' sums pass through the first words of hw, cleared afterwards.
  {
    constexpr int kPer = kSplitMaxBuckets / kThreads;   // 16
    int32_t* wsum = reinterpret_cast<int32_t*>(hw);
    int32_t tv[kPer], pv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = min(kPer * tid + u, nb - 1);
      tv[u] = bs[i];
      pv[u] = pre[i];
    }
    int32_t mine = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) mine += kPer * tid + u < nb ? tv[u] : 0;
    // exclusive prefix of the per-thread sums over the workgroup
    int32_t inc = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int32_t o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    int32_t acc = inc - mine;
#pragma unroll
    for (int w2 = 0; w2 < kSplitWaves; ++w2) acc += w2 < w ? wsum[w2] : 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = kPer * tid + u;
      if (i < nb) run[i] = acc + pv[u];
      acc += i < nb ? tv[u] : 0;
    }
  }
  __syncthreads();   // the waves' sums are read
  for (int i = tid; i < kSplitWaves * nb / 2; i += kThreads) hw[i] = 0u;
  __syncthreads();

  // pass 1: this wave's count of every bucket (nb is even, so the wave's
  // table starts on a word: bucket k of wave w is half k % 2 of word
  // (w * nb + k) / 2)
  for (int c0 = wlo; c0 < whi; c0 += kWave * kScatterBatches) {
    int key[kScatterBatches];
#pragma unroll
    for (int b = 0; b < kScatterBatches; ++b) key[b] = bk[min(c0 + b * kWave + lane, whi - 1)];
#pragma unroll
    for (int b = 0; b < kScatterBatches; ++b) {
      if (c0 + b * kWave + lane < whi) {
        const int k = clamp_bucket(key[b], nb);
        atomicAdd(&hw[(w * nb + k) >> 1], 1u << (16 * (k & 1)));
      }
    }
  }
  __syncthreads();
  // the counts become offsets: wave w's run of bucket b starts after the
  // keys of b in the waves before it
  for (int b = tid; b < nb; b += kThreads) {
    const uint16_t* h0 = reinterpret_cast<const uint16_t*>(hw);
    uint16_t* hm = reinterpret_cast<uint16_t*>(hw);
    int acc = 0;
#pragma unroll
    for (int w2 = 0; w2 < kSplitWaves; ++w2) {
      const int c = h0[w2 * nb + b];
      hm[w2 * nb + b] = (uint16_t)acc;
      acc += c;
    }
  }
  __syncthreads();

  // pass 2: ranks in position order and the scatter
  for (int c0 = wlo; c0 < whi; c0 += kWave * kScatterBatches) {
    int key[kScatterBatches];
#pragma unroll
    for (int b = 0; b < kScatterBatches; ++b) key[b] = bk[min(c0 + b * kWave + lane, whi - 1)];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int b = 0; b < kScatterBatches; ++b) {
      const int i0 = c0 + b * kWave;
      if (i0 >= whi) break;
      const int i = i0 + lane;
      const bool valid = i < whi;
      const int k = valid ? clamp_bucket(key[b], nb) : 0;
      uint64_t peers = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (k >> bit) & 1;
        const uint64_t ones = __ballot(set);
        peers &= set ? ones : ~ones;
      }
      const int off = valid ? (int)h16[k] : 0;
      const int32_t start = valid ? run[k] : 0;
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
      const int n = __popcll(peers);
      __builtin_amdgcn_wave_barrier();
      if (valid && rank == n - 1) h16[k] = (uint16_t)(off + n);
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        const int32_t slot = start + off + rank;
        pm[slot] = i;
        ip[i] = slot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide tiles (B <= 2048).  One workgroup of W waves per (segment, tile of
// W * 64 * nbat keys, nbat <= 32 batches of 64 per wave, at most 16,384 keys).
//   1. each wave ranks its own nbat batches in position order: equal keys of
//      a batch are found through the wave's own per-bucket LDS masks, and a
//      key's rank is the wave's running count of its bucket plus its rank
//      among the equal keys of lower lanes;
//   2. the per-wave counts become per-wave exclusive prefixes; the tile's
//      bucket starts are a block scan of the tile's counts, and the global
//      slot of the tile's first key of bucket b (bucket base plus the counts
//      of the segment's earlier tiles, both from the count table) is kept
//      as delta[b] = that slot - start[b];
//   3. every key's tile-local sorted index q goes into LDS (stage[q] = its
//      tile-local position and bucket), and inv_perm is written at once, in
//      position order (coalesced);
//   4. perm is written from the stage in sorted order: consecutive threads
//      write consecutive slots wherever a bucket's run in the tile continues,
//      instead of one scattered 4-byte store per key.
// The count table comes from sort_wide_count_kernel (one launch before).
// NBMAX: the largest bucket count of the instance (per-wave tables in LDS).
constexpr int kWideMaxBatches = 32;
constexpr int kWidePosBits = 14;          // tile-local positions < 2^14
constexpr int kWideMaxTile = 1 << kWidePosBits;
constexpr int kWideCountThreads = 1024;

__global__ __launch_bounds__(kWideCountThreads) void sort_wide_count_kernel(
    const int32_t* __restrict__ buckets, int32_t* __restrict__ cnt, int L, int nb, int tile,
    int ntiles) {
  __shared__ int32_t hist[kWideMaxBuckets];
  const int64_t seg = blockIdx.x / ntiles;
  const int t = blockIdx.x % ntiles;
  for (int i = threadIdx.x; i < nb; i += kWideCountThreads) hist[i] = 0;
  __syncthreads();
  const int lo = t * tile;
  const int hi = min(L, lo + tile);
  const int32_t* bk = buckets + seg * L;
  // sixteen keys per thread requested before any is counted (clamped indices)
  for (int i0 = lo; i0 < hi; i0 += kWideCountThreads * 16) {
    int32_t k[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) k[u] = bk[min(i0 + kWideCountThreads * u + (int)threadIdx.x, hi - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (i0 + kWideCountThreads * u + (int)threadIdx.x < hi)
        atomicAdd(&hist[clamp_bucket(k[u], nb)], 1);
  }
  __syncthreads();
  int32_t* out = cnt + (seg * ntiles + t) * (int64_t)nb;
  for (int i = threadIdx.x; i < nb; i += kWideCountThreads) out[i] = hist[i];
}

__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

template <int W, int NBMAX>
__global__ __launch_bounds__(kWave * W) void sort_wide_scatter_kernel(
    const int32_t* __restrict__ buckets, const int32_t* __restrict__ cnt,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm, int L, int nb, int tile,
    int ntiles, int nbat) {
  constexpr int kNbMax = NBMAX;                    // largest bucket count
  constexpr int kThreads = kWave * W;
  // masks [W][kNbMax] during ranking; afterwards the stage [tile] (aliased)
  __shared__ __attribute__((aligned(16))) uint64_t region[W * kNbMax];
  __shared__ int32_t cw_all[W * kNbMax];            // per-wave counts, then prefixes
  __shared__ int32_t bstart[kNbMax], delta[kNbMax], total[kNbMax];
  __shared__ int32_t part[2 * W];
  // the stage (tile-local sorted positions) fits the mask region: tiles of
  // at most 2 * W * NBMAX keys

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid >> 6;
  // each XCD takes a contiguous range of (segment, tile): the runs of
  // neighbouring tiles of one segment fill the same perm lines in one L2
  const int64_t blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int64_t seg = blk / ntiles;
  const int t = (int)(blk % ntiles);
  const int lo = t * tile;
  const int hi = min(L, lo + tile);
  const int32_t* bk = buckets + seg * L;
  uint64_t* mask = region + w * nb;
  int32_t* cw = cw_all + w * nb;
  for (int i = lane; i < nb; i += kWave) {
    mask[i] = 0;
    cw[i] = 0;
  }
  // batch j of wave w: tile positions (w * nbat + j) * 64 + lane; the loads
  // are issued together (clamped into the tile; a batch past the tile's end
  // is skipped whole, L being a multiple of 64)
  const int wlo = lo + w * nbat * kWave;
  int key[kWideMaxBatches], rk[kWideMaxBatches];
#pragma unroll
  for (int j = 0; j < kWideMaxBatches; ++j)
    key[j] = bk[min(wlo + min(j, nbat - 1) * kWave + lane, hi - 1)];
#pragma unroll
  for (int j = 0; j < kWideMaxBatches; ++j) key[j] = clamp_bucket(key[j], nb);
  __builtin_amdgcn_wave_barrier();

  // 1. ranks inside the wave, batch by batch in position order.  A wave's LDS
  // operations take effect in order, so each lane's read of its bucket's mask
  // sees the bits of the whole batch.
#pragma unroll
  for (int j = 0; j < kWideMaxBatches; ++j) {
    if (j >= nbat || wlo + j * kWave >= hi) continue;   // uniform
    const int k = key[j];
    __hip_atomic_fetch_or(&mask[k], 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __builtin_amdgcn_wave_barrier();
    const uint64_t peers = __hip_atomic_load(&mask[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int c = cw[k];
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
    const int n = __popcll(peers);
    rk[j] = c + rank;
    __builtin_amdgcn_wave_barrier();
    if (rank == n - 1) {
      cw[k] = c + n;
      __hip_atomic_store(&mask[k], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // 2. thread tid owns buckets [tid * per, tid * per + per)
  const int per = (nb + kThreads - 1) / kThreads;
  const int32_t* ct = cnt + seg * (int64_t)ntiles * nb;
  int my_tc = 0, my_tot = 0;
  for (int q = 0; q < per; ++q) {
    const int b = tid * per + q;
    if (b >= nb) break;
    int run = 0;
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) {
      const int v = cw_all[w2 * nb + b];
      cw_all[w2 * nb + b] = run;
      run += v;
    }
    // the counts of b in every tile of the segment, eight loads in flight
    int pre = 0, tot = 0;
    for (int t0 = 0; t0 < ntiles; t0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ct[(int64_t)min(t0 + u, ntiles - 1) * nb + b];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t2 = t0 + u;
        pre += t2 < t ? v[u] : 0;
        tot += t2 < ntiles ? v[u] : 0;
      }
    }
    bstart[b] = run;   // for now: the tile's count of b
    delta[b] = pre;    // for now: the counts of b in the segment's earlier tiles
    total[b] = tot;
    my_tc += run;
    my_tot += tot;
  }
  const int inc_tc = wave_inclusive_sum(my_tc);
  const int inc_tot = wave_inclusive_sum(my_tot);
  if (lane == kWave - 1) {
    part[w] = inc_tc;
    part[W + w] = inc_tot;
  }
  __syncthreads();
  int run_tc = inc_tc - my_tc, run_tot = inc_tot - my_tot;
#pragma unroll
  for (int w2 = 0; w2 < W; ++w2) {
    if (w2 < w) {
      run_tc += part[w2];
      run_tot += part[W + w2];
    }
  }
  for (int q = 0; q < per; ++q) {
    const int b = tid * per + q;
    if (b >= nb) break;
    const int c = bstart[b], pre = delta[b], tot = total[b];
    bstart[b] = run_tc;
    delta[b] = run_tot + pre - run_tc;   // bucket base + earlier tiles - tile start
    run_tc += c;
    run_tot += tot;
  }
  __syncthreads();

  // 3. tile-local sorted index of every key: stage it, write inv_perm
  int32_t* stage = reinterpret_cast<int32_t*>(region);
  int32_t* ip = inv_perm + seg * L;
#pragma unroll
  for (int j = 0; j < kWideMaxBatches; ++j) {
    if (j >= nbat || wlo + j * kWave >= hi) continue;   // uniform
    const int k = key[j];
    const int q = bstart[k] + cw[k] + rk[j];
    const int i = wlo + j * kWave + lane;
    stage[q] = (i - lo) | (k << kWidePosBits);
    ip[i] = delta[k] + q;
  }
  __syncthreads();

  // 4. perm in sorted order, runs of consecutive slots per bucket
  int32_t* pm = perm + seg * L;
  const int n = hi - lo;
  for (int q0 = 0; q0 < n; q0 += kThreads * 4) {
    int e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = stage[min(q0 + kThreads * u + tid, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + kThreads * u + tid;
      if (q < n) {
        const int k = e[u] >> kWidePosBits;
        pm[clamp_index(delta[k] + q, L)] = lo + (e[u] & (kWideMaxTile - 1));
      }
    }
  }
}

template <int W, int NBMAX>
static void launch_wide_scatter(dim3 grid, hipStream_t stream, const int32_t* buckets,
                                const int32_t* cnt, int32_t* perm, int32_t* inv_perm, int L,
                                int nb, int tile, int ntiles, int nbat) {
  hipLaunchKernelGGL((sort_wide_scatter_kernel<W, NBMAX>), grid, dim3(kWave * W), 0, stream,
                     buckets, cnt, perm, inv_perm, L, nb, tile, ntiles, nbat);
}

hipError_t launch_sort(const Shape& s, const int32_t* buckets, int32_t* perm, int32_t* inv_perm,
                       void* workspace, hipStream_t stream) {
  const int64_t S = s.segments();
  const int tile = sort_tile(s);
  const int ntiles = (int)sort_tiles(s);
  const int nb = s.buckets;
  int32_t* cnt = static_cast<int32_t*>(workspace);
  if (nb <= kWideMaxBuckets) {
    const WidePlan p = wide_plan(s);
    const dim3 grid((unsigned)(S * ntiles));
    hipLaunchKernelGGL(sort_wide_count_kernel, grid, dim3(kWideCountThreads), 0, stream, buckets,
                       cnt, s.len, nb, tile, ntiles);
    if (p.nbmax == 256 && p.waves == 8)
      launch_wide_scatter<8, 256>(grid, stream, buckets, cnt, perm, inv_perm, s.len, nb, tile,
                                  ntiles, p.nbat);
    else if (p.nbmax == 256)
      launch_wide_scatter<4, 256>(grid, stream, buckets, cnt, perm, inv_perm, s.len, nb, tile,
                                  ntiles, p.nbat);
    else if (p.nbmax == 1024 && p.waves == 8)
      launch_wide_scatter<8, 1024>(grid, stream, buckets, cnt, perm, inv_perm, s.len, nb, tile,
                                   ntiles, p.nbat);
    else if (p.nbmax == 1024)
      launch_wide_scatter<4, 1024>(grid, stream, buckets, cnt, perm, inv_perm, s.len, nb, tile,
                                   ntiles, p.nbat);
    else
      launch_wide_scatter<4, 2048>(grid, stream, buckets, cnt, perm, inv_perm, s.len, nb, tile,
                                   ntiles, p.nbat);
    return hipGetLastError();
  }
  int nbits = 0;
  while ((1 << nbits) < nb) ++nbits;
  const size_t cnt_bytes = ((size_t)S * ntiles * nb * sizeof(int32_t) + 255) & ~(size_t)255;
  int32_t* base = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + cnt_bytes);
  const size_t lds = (size_t)nb * sizeof(int32_t);

  // the eight-wave scatter computes the bucket bases from the totals itself
  const bool split = nb <= kSplitMaxBuckets && tile >= kSplitWaves * kWave;
  // one workgroup per segment pays off while a segment is short: a long one
  // is counted faster by a workgroup per tile
  if (!split && (int64_t)ntiles * nb <= kPrefixLdsInts && s.len <= kPrefixMaxLen) {
    hipLaunchKernelGGL(sort_prefix_kernel, dim3((unsigned)S), dim3(kPrefixThreads), 0, stream,
                       buckets, cnt, base, s.len, nb, tile, ntiles);
  } else {
    hipLaunchKernelGGL(sort_count_kernel, dim3((unsigned)(S * ntiles)), dim3(256), lds, stream,
                       buckets, cnt, s.len, nb, tile, ntiles);
    // one thread per (segment, bucket), in launch pieces
    const int64_t nbins = S * nb;
    const int64_t nblk = (nbins + 255) / 256;
    for (int64_t b0 = 0; b0 < nblk; b0 += kMaxBlocks)
      hipLaunchKernelGGL(sort_scan_tiles_kernel, dim3((unsigned)std::min(kMaxBlocks, nblk - b0)),
                         dim3(256), 0, stream, cnt, base, nb, ntiles, nbins, b0);
    if (!split)
      hipLaunchKernelGGL(sort_scan_bins_kernel, dim3((unsigned)S), dim3(1024), 0, stream, base,
                         nb);
  }
  if (split)
    hipLaunchKernelGGL(sort_scatter_split_kernel, dim3((unsigned)(S * ntiles)),
                       dim3(kWave * kSplitWaves), 0, stream, buckets, cnt, base, perm, inv_perm,
                       s.len, nb, nbits, tile, ntiles);
  else
    hipLaunchKernelGGL(sort_scatter_kernel, dim3((unsigned)(S * ntiles)), dim3(64), lds, stream,
                       buckets, cnt, base, perm, inv_perm, s.len, nb, nbits, tile, ntiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// The sort's count tables in the library's own device memory, for callers
// that cannot allocate.  One array per GPU, alive until the process ends;
// every call on that GPU shares it, so calls that overlap on one GPU race.
// Its contents on entry do not matter: the count pass writes every table
// entry the scatter reads.  In host code `scratch` names a host-side stand-in:
// kernels are given the device address looked up once per device below.
constexpr size_t kStaticSortScratch = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticSortScratch];

size_t static_sort_scratch_bytes() { return kStaticSortScratch; }

hipError_t static_sort_scratch(int device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != device ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (!p) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

}  // namespace lsh
