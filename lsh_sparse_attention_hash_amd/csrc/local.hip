// local.hip -- local chunked self-attention, the method's attention without
// hashing (Reformer overview page "The Reformer - Pushing the limits of
// language modeling", sections "Approach / What changed" and "Takeaways": the
// sequence is cut into chunks of length l_c and each chunk also attends to a
// configurable number of chunks before and after it).  Scores, masks and the
// empty-set rule are those of the LSH attention (Q = K with unit-length keys,
// 1/sqrt(d), causal by position, self-mask, y_i = v_i when nothing is left).
//
// One workgroup per (batch, head, query chunk c): the 64 queries stay in
// registers and the key chunks max(0, c - before) .. min(C - 1, c + after)
// (.. c when causal) stream through LDS, the next one in flight while the
// current one is computed, under an online softmax.  Neighbouring query
// chunks share key chunks, so workgroups are mapped so that each XCD walks a
// contiguous range of chunks and the re-reads hit its L2.
//
// bf16: S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 as in the
// bucketed attention (one query per lane column; a fifth tile of ones gives
// the row sums of the rounded probabilities).  fp32: one thread per query.
#include <math.h>

#include <algorithm>

#include "lsh_device.h"
#include "lsh_launch.h"

namespace lsh {

// Sum over each group of eight lanes (8m .. 8m + 7) by DPP exchanges inside
// the lanes' row (lane ^ 1 and lane ^ 2 by quad permutes, then the other
// quad of the eight through the half-row mirror): the additions pair the
// lanes as lane ^ 1, ^ 2, ^ 4 would, so the sums are the same bits, with no
// LDS permute.
__device__ __forceinline__ float sum8_lanes(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

// Maximum of lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane groups):
// ds_swizzle for lane ^ 16 inside each half, the half swap for lane ^ 32.
__device__ __forceinline__ float max4_groups(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
  return fmaxf(v, other_half(v));
}

constexpr int kKeyStride = 72;   // bf16 per key row in LDS (144 B)
constexpr int kVtRowDw = 36;     // dwords per V^T row: 32 key pairs + 4 pad
constexpr float kLog2eL = 1.4426950408889634f;
constexpr float kLn2L = 0.6931471805599453f;
constexpr float kEps = 1e-6f;

struct LocalArgs {
  const void* qk;
  const void* v;
  float* y;
  float* lse;
  int L, nchunks, before, after;
  int64_t blk0;   // first block of this launch piece
};

struct LocalLds {
  uint16_t xs[kChunk * kKeyStride];
  uint32_t vt[kHeadDim * kVtRowDw];   // V^T, dword column XOR-swizzled by 8 * ((d >> 4) & 3)
  float kinv[kChunk];                 // log2(e) / (max(|x_j|, eps) * sqrt(d))
};

// Thread t stages keys 2*(t/8), 2*(t/8)+1 of a chunk, 16-byte column block t%8.
struct KeyRegs {
  uint4 xa, xc, va, vc;
};

__device__ __forceinline__ void gather_keys(KeyRegs& g, const uint16_t* xb, const uint16_t* vb,
                                            int kc) {
  const int dblk = threadIdx.x & 7;
  const size_t r0 = (size_t)kc * kChunk + 2 * (threadIdx.x >> 3);
  g.xa = load16(xb + r0 * kHeadDim + 8 * dblk);
  g.xc = load16(xb + (r0 + 1) * kHeadDim + 8 * dblk);
  g.va = load16(vb + r0 * kHeadDim + 8 * dblk);
  g.vc = load16(vb + (r0 + 1) * kHeadDim + 8 * dblk);
}

__device__ __forceinline__ void commit_keys(LocalLds& sm, const KeyRegs& g) {
  const int p = threadIdx.x >> 3;   // key pair
  const int dblk = threadIdx.x & 7;
  store16(&sm.xs[(2 * p) * kKeyStride + 8 * dblk], g.xa);
  store16(&sm.xs[(2 * p + 1) * kKeyStride + 8 * dblk], g.xc);
  const uint32_t wa[4] = {g.va.x, g.va.y, g.va.z, g.va.w};
  const uint32_t wc[4] = {g.vc.x, g.vc.y, g.vc.z, g.vc.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int d0 = 8 * dblk + 2 * e;
    sm.vt[d0 * kVtRowDw + (p ^ (8 * ((d0 >> 4) & 3)))] = (wa[e] & 0xffffu) | (wc[e] << 16);
    sm.vt[(d0 + 1) * kVtRowDw + (p ^ (8 * (((d0 + 1) >> 4) & 3)))] =
        (wa[e] >> 16) | (wc[e] & 0xffff0000u);
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
  sa = sum8_lanes(sa);
  sc = sum8_lanes(sc);
  if (dblk == 0) {
    sm.kinv[2 * p] = (kLog2eL / 8.0f) * __builtin_amdgcn_rsqf(fmaxf(sa, kEps * kEps));
    sm.kinv[2 * p + 1] = (kLog2eL / 8.0f) * __builtin_amdgcn_rsqf(fmaxf(sc, kEps * kEps));
  }
}

// Online-softmax state of the lane's query: running max (log2 units) and the
// O^T accumulators (tiles 0..3: d = 16*dt + 4*g + i; tile 4: row sum).
struct QueryState {
  float m;
  f32x4 o[5];
};

template <bool CAUSAL, bool SELF>
__device__ __forceinline__ void attend_keys(const LocalLds& sm, const bf16x8 (&qf)[2],
                                            QueryState& st, bool diag, int qi) {
  const int lane = lane_id();
  const int g = lane >> 4;
  const int ql = lane & 15;
  // s[t][i]: key 16t + 4g + i of the chunk, log2-scaled
  float s[4][4];
  float cm = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 kf = as_bf16x8(load16(&sm.xs[(16 * t + ql) * kKeyStride + 8 * g + 32 * ks]));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], acc, 0, 0, 0);
    }
    const float4 kv = *reinterpret_cast<const float4*>(&sm.kinv[16 * t + 4 * g]);
    const float kva[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 16 * t + 4 * g + i;
      bool ok = true;
      if (CAUSAL) ok = !diag || key <= qi;
      if (SELF) ok = ok && !(diag && key == qi);
      s[t][i] = ok ? acc[i] * kva[i] : -INFINITY;
      cm = fmaxf(cm, s[t][i]);
    }
  }
  cm = max4_groups(cm);
  const float mn = fmaxf(st.m, cm);
  const float msafe = mn == -INFINITY ? 0.f : mn;
  const float scale = __builtin_amdgcn_exp2f(st.m - msafe);   // 0 while nothing was kept
  st.m = mn;
#pragma unroll
  for (int dt = 0; dt < 5; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) st.o[dt][i] *= scale;

  uint32_t pw[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const bf16x2 pr = {(__bf16)__builtin_amdgcn_exp2f(s[t][i] - msafe),
                         (__bf16)__builtin_amdgcn_exp2f(s[t][i + 1] - msafe)};
      pw[t][i >> 1] = __builtin_bit_cast(uint32_t, pr);
    }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u,
                                                            0x3f803f80u));
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    // MFMA contraction index 8g + j <-> key 32*k2 + 16*(j/4) + 4g + j%4
    const bf16x8 pb = __builtin_bit_cast(
        bf16x8, make_uint4(pw[2 * k2][0], pw[2 * k2][1], pw[2 * k2 + 1][0], pw[2 * k2 + 1][1]));
    const int c0 = 16 * k2 + 2 * g;   // key-pair (dword) columns of keys 32k2 + 4g.. and +16
    const int c1 = c0 + 8;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint32_t* vrow = &sm.vt[(16 * dt + ql) * kVtRowDw];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (c0 ^ (8 * dt)));
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (c1 ^ (8 * dt)));
      const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, st.o[dt], 0, 0, 0);
    }
    st.o[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, st.o[4], 0, 0, 0);
  }
}

// NPRE = 1: any window, the next key chunk in flight during the current one.
// NPRE = 3: windows of at most three chunks, all of them requested at once, so
// the workgroup waits on memory once instead of once per chunk.
template <bool CAUSAL, bool SELF, int NPRE>
__global__ __launch_bounds__(256) void local_bf16_kernel(LocalArgs a) {
  __shared__ __attribute__((aligned(16))) LocalLds sm;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int ql = lane & 15;
  const int64_t blk = a.blk0 + xcd_logical_block(blockIdx.x, gridDim.x);
  const int64_t bh = blk / a.nchunks;
  const int c = (int)(blk % a.nchunks);
  const int k0 = c - min(c, a.before);
  const int k1 = CAUSAL ? c : c + min(a.nchunks - 1 - c, a.after);
  const uint16_t* xb = static_cast<const uint16_t*>(a.qk) + bh * (int64_t)a.L * kHeadDim;
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + bh * (int64_t)a.L * kHeadDim;

  const int qi = 16 * wave + ql;                 // query row inside the chunk
  const int64_t qrow = (int64_t)c * kChunk + qi;
  bf16x8 qf[2];                                  // B operand Q^T: x_q[8g + 32ks .. +7]
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) qf[ks] = as_bf16x8(load16(xb + qrow * kHeadDim + 8 * g + 32 * ks));

  QueryState st;
  st.m = -INFINITY;
#pragma unroll
  for (int dt = 0; dt < 5; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (NPRE == 1) {
    KeyRegs kr;
    gather_keys(kr, xb, vb, k0);
    for (int kc = k0; kc <= k1; ++kc) {
      commit_keys(sm, kr);
      if (kc < k1) gather_keys(kr, xb, vb, kc + 1);   // in flight during the compute
      __syncthreads();
      attend_keys<CAUSAL, SELF>(sm, qf, st, kc == c, qi);
      __syncthreads();
    }
  } else {
    // unconditional (chunks past the window repeat the last one, unused), so
    // that the first chunk is committed as soon as its own rows are in
    KeyRegs kr[NPRE];
#pragma unroll
    for (int i = 0; i < NPRE; ++i) gather_keys(kr[i], xb, vb, min(k0 + i, k1));
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      if (k0 + i > k1) break;
      commit_keys(sm, kr[i]);
      __syncthreads();
      attend_keys<CAUSAL, SELF>(sm, qf, st, k0 + i == c, qi);
      __syncthreads();
    }
  }

  const float sum = st.o[4][0];
  float* yrow = a.y + (bh * a.L + qrow) * kHeadDim;
  if (sum > 0.f) {
    const float inv = __builtin_amdgcn_rcpf(sum);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<float4*>(yrow + 16 * dt + 4 * g) =
          make_float4(st.o[dt][0] * inv, st.o[dt][1] * inv, st.o[dt][2] * inv, st.o[dt][3] * inv);
  } else {
    // no key left (only with the self-mask): the token keeps its own value
    const uint16_t* vrow = vb + qrow * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint2 w = *reinterpret_cast<const uint2*>(vrow + 16 * dt + 4 * g);
      *reinterpret_cast<float4*>(yrow + 16 * dt + 4 * g) =
          make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
    }
  }
  if (g == 0)
    a.lse[bh * a.L + qrow] = sum > 0.f ? (st.m + __builtin_amdgcn_logf(sum)) * kLn2L : -INFINITY;
}

// ------------------------------------------------------------------- fp32
// One wave per (batch, head, query chunk); lane q is query q of the chunk.
// Key chunks are staged 64 keys at a time; the softmax runs online in fp32.
__global__ __launch_bounds__(64) void local_f32_kernel(LocalArgs a, int causal, int self_mask) {
  __shared__ float xw[kChunk][kHeadDim];
  __shared__ float vw[kChunk][kHeadDim];
  __shared__ float kinv[kChunk];
  const int lane = lane_id();
  const int64_t blk = a.blk0 + blockIdx.x;
  const int64_t bh = blk / a.nchunks;
  const int c = (int)(blk % a.nchunks);
  const int k0 = c - min(c, a.before);
  const int k1 = causal ? c : c + min(a.nchunks - 1 - c, a.after);
  const float* xb = static_cast<const float*>(a.qk) + bh * (int64_t)a.L * kHeadDim;
  const float* vb = static_cast<const float*>(a.v) + bh * (int64_t)a.L * kHeadDim;
  const int qp = c * kChunk + lane;
  float xq[kHeadDim];
#pragma unroll
  for (int k = 0; k < kHeadDim; ++k) xq[k] = xb[(int64_t)qp * kHeadDim + k];
  float m = -INFINITY, l = 0.f, o[kHeadDim];
#pragma unroll
  for (int k = 0; k < kHeadDim; ++k) o[k] = 0.f;

  for (int kc = k0; kc <= k1; ++kc) {
    __syncthreads();
    const int pos = kc * kChunk + lane;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kHeadDim; ++k) {
      const float xv = xb[(int64_t)pos * kHeadDim + k];
      xw[lane][k] = xv;
      vw[lane][k] = vb[(int64_t)pos * kHeadDim + k];
      ss += xv * xv;
    }
    kinv[lane] = 1.0f / (fmaxf(sqrtf(ss), kEps) * 8.0f);
    __syncthreads();
    for (int kk = 0; kk < kChunk; ++kk) {
      const int kp = kc * kChunk + kk;
      if ((causal && kp > qp) || (self_mask && kp == qp)) continue;
      float dot = 0.f;
#pragma unroll
      for (int k = 0; k < kHeadDim; ++k) dot = fmaf(xq[k], xw[kk][k], dot);
      const float sc = dot * kinv[kk];
      if (sc > m) {
        const float f = expf(m - sc);
        l *= f;
#pragma unroll
        for (int k = 0; k < kHeadDim; ++k) o[k] *= f;
        m = sc;
      }
      const float p = expf(sc - m);
      l += p;
#pragma unroll
      for (int k = 0; k < kHeadDim; ++k) o[k] = fmaf(p, vw[kk][k], o[k]);
    }
  }
  float* yrow = a.y + (bh * a.L + qp) * kHeadDim;
  if (l > 0.f) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int k = 0; k < kHeadDim; k += 4)
      *reinterpret_cast<float4*>(yrow + k) =
          make_float4(o[k] * inv, o[k + 1] * inv, o[k + 2] * inv, o[k + 3] * inv);
  } else {
#pragma unroll
    for (int k = 0; k < kHeadDim; k += 4)
      *reinterpret_cast<float4*>(yrow + k) =
          *reinterpret_cast<const float4*>(vb + (int64_t)qp * kHeadDim + k);
  }
  a.lse[bh * a.L + qp] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int NPRE>
static void launch_local_bf16(const Shape& s, const LocalArgs& a, unsigned grid,
                              hipStream_t stream) {
  if (s.causal && s.self_mask)
    hipLaunchKernelGGL((local_bf16_kernel<true, true, NPRE>), dim3(grid), dim3(256), 0, stream, a);
  else if (s.causal)
    hipLaunchKernelGGL((local_bf16_kernel<true, false, NPRE>), dim3(grid), dim3(256), 0, stream, a);
  else if (s.self_mask)
    hipLaunchKernelGGL((local_bf16_kernel<false, true, NPRE>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((local_bf16_kernel<false, false, NPRE>), dim3(grid), dim3(256), 0, stream, a);
}

hipError_t launch_local(const Shape& s, int before, int after, const void* qk, const void* v,
                        float* y, float* lse, hipStream_t stream) {
  LocalArgs a;
  a.qk = qk;
  a.v = v;
  a.y = y;
  a.lse = lse;
  a.L = s.len;
  a.nchunks = s.len / kChunk;
  // a window wider than the sequence is the whole sequence
  a.before = before < a.nchunks ? before : a.nchunks;
  a.after = after < a.nchunks ? after : a.nchunks;
  const int64_t nblk = s.token_heads() / kChunk;
  for (int64_t b0 = 0; b0 < nblk; b0 += kMaxBlocks) {
    a.blk0 = b0;
    const unsigned grid = (unsigned)std::min(kMaxBlocks, nblk - b0);
    if (!s.bf16)
      hipLaunchKernelGGL(local_f32_kernel, dim3(grid), dim3(64), 0, stream, a, s.causal,
                         s.self_mask);
    else if (a.before + 1 + (s.causal ? 0 : a.after) <= 3)
      launch_local_bf16<3>(s, a, grid, stream);
    else
      launch_local_bf16<1>(s, a, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace lsh
