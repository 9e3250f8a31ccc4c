// sort.hip -- stable counting sort of every (batch, head, round) segment by
// bucket id (Reformer study note, section "Sorting and Chunking": tokens are
// sorted by hash bucket so each bucket becomes contiguous).  Because positions
// enter in increasing order and the scatter is stable, the result is the
// order of the unique key (bucket, original position).
//
// Four launches per call (two for segments of at most 16,384 tokens whose
// tile histograms fit in LDS: prefix, one workgroup per segment, does the
// first three):
//   count    one workgroup per (segment, tile): LDS histogram of the tile
//   scan_t   one thread per (segment, bucket): exclusive prefix over tiles
//   scan_b   one workgroup per segment: exclusive prefix over bucket totals
//   scatter  one wave per (segment, tile): walks the tile in order, 64 keys
//            at a time; equal keys inside a batch are ranked by lane (found
//            through per-bucket LDS masks, or ballots over the key bits for
//            B > 2048), so the scatter is stable.
// Workspace: cnt[S][tiles][B] (counts, then tile prefixes) and base[S][B].
#include <mutex>

#include "lsh_device.h"
#include "lsh_launch.h"

namespace lsh {

int sort_tile(const Shape& s) {
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
                                                             int ntiles, int64_t nbins_total) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

// One wave per (segment, tile).  The tile's keys are first loaded into
// registers (kScatterBatches loads in flight per lane), then ranked 64 at a
// time in position order; each key's slot is its bucket's running offset (LDS)
// plus its rank among the equal keys of lower lanes.  The lanes holding equal
// keys are found
//   MASK:  through LDS -- every lane ORs its lane bit into its bucket's 64-bit
//          mask, reads the mask back (a wave's LDS operations take effect in
//          order, so the read sees the whole batch), and the group's last lane
//          advances the bucket's offset and clears the mask (B <= 2048);
//   else:  by intersecting the ballots of every key bit.
constexpr int kScatterBatches = 32;   // keys taken 32 batches of 64 at a time
constexpr int kMaskMatchMaxBuckets = 2048;

template <bool MASK>
__global__ __launch_bounds__(64) void sort_scatter_kernel(
    const int32_t* __restrict__ buckets, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ base, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int L, int nb, int nbits, int tile, int ntiles) {
  extern __shared__ uint64_t smem[];
  uint64_t* mask = smem;                                              // [nb] (MASK)
  int32_t* run = MASK ? reinterpret_cast<int32_t*>(smem + nb) : reinterpret_cast<int32_t*>(smem);
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
      if (i < nb) {
        run[i] = bv[u] + pv[u];
        if (MASK) mask[i] = 0;
      }
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
      uint64_t peers;
      int32_t start = 0;
      if (MASK) {
        if (valid) __hip_atomic_fetch_or(&mask[k], 1ull << lane, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP);
        __builtin_amdgcn_wave_barrier();
        peers = 0;
        if (valid) {
          peers = __hip_atomic_load(&mask[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          start = run[k];
        }
      } else {
        peers = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
          const bool set = (k >> bit) & 1;
          const uint64_t ones = __ballot(set);
          peers &= set ? ones : ~ones;
        }
        start = valid ? run[k] : 0;
      }
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
      const int n = __popcll(peers);
      __builtin_amdgcn_wave_barrier();
      if (valid && rank == n - 1) {
        run[k] = start + n;
        if (MASK) __hip_atomic_store(&mask[k], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        const int32_t slot = start + rank;
        pm[slot] = i;
        ip[i] = slot;
      }
    }
  }
}

hipError_t launch_sort(const Shape& s, const int32_t* buckets, int32_t* perm, int32_t* inv_perm,
                       void* workspace, hipStream_t stream) {
  const int64_t S = s.segments();
  const int tile = sort_tile(s);
  const int ntiles = (int)sort_tiles(s);
  const int nb = s.buckets;
  int nbits = 0;
  while ((1 << nbits) < nb) ++nbits;
  int32_t* cnt = static_cast<int32_t*>(workspace);
  const size_t cnt_bytes = ((size_t)S * ntiles * nb * sizeof(int32_t) + 255) & ~(size_t)255;
  int32_t* base = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + cnt_bytes);
  const size_t lds = (size_t)nb * sizeof(int32_t);

  // one workgroup per segment pays off while a segment is short: a long one
  // is counted faster by a workgroup per tile
  if ((int64_t)ntiles * nb <= kPrefixLdsInts && s.len <= kPrefixMaxLen) {
    hipLaunchKernelGGL(sort_prefix_kernel, dim3((unsigned)S), dim3(kPrefixThreads), 0, stream,
                       buckets, cnt, base, s.len, nb, tile, ntiles);
  } else {
    hipLaunchKernelGGL(sort_count_kernel, dim3((unsigned)(S * ntiles)), dim3(256), lds, stream,
                       buckets, cnt, s.len, nb, tile, ntiles);
    const int64_t nbins = S * nb;
    hipLaunchKernelGGL(sort_scan_tiles_kernel, dim3((unsigned)((nbins + 255) / 256)), dim3(256),
                       0, stream, cnt, base, nb, ntiles, nbins);
    hipLaunchKernelGGL(sort_scan_bins_kernel, dim3((unsigned)S), dim3(1024), 0, stream, base, nb);
  }
  if (nb <= kMaskMatchMaxBuckets)
    hipLaunchKernelGGL(sort_scatter_kernel<true>, dim3((unsigned)(S * ntiles)), dim3(64),
                       (size_t)nb * (sizeof(uint64_t) + sizeof(int32_t)), stream, buckets, cnt,
                       base, perm, inv_perm, s.len, nb, nbits, tile, ntiles);
  else
    hipLaunchKernelGGL(sort_scatter_kernel<false>, dim3((unsigned)(S * ntiles)), dim3(64), lds,
                       stream, buckets, cnt, base, perm, inv_perm, s.len, nb, nbits, tile, ntiles);
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
