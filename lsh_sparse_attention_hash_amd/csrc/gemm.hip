// gemm.hip -- the dense maps of the reversible layer (Reformer study note,
// "Reversible Residual Layers": y1 = x1 + F(x2), y2 = x2 + G(y1); "Chunked
// Feed-Forward Computation": G(x) = W2 ReLU(W1 x + b1) + b2 token by token):
// C[m][n] = sum_k A[m][k] W[n][k] on v_mfma_f32_32x32x16_bf16 with fused
// epilogues.
//
// A is bf16 or fp32 (rounded to bf16, nearest-even, as it is staged), in rows
// [M][lda] or, for the attention output, as heads [b][H][L][64] read as the
// concatenation [b*L][H*64] (fp32, or bf16 inside the reversible layer).  W is bf16, one row per output feature ([N][K]),
// so both operands are K-contiguous: every MFMA fragment is one 16-byte load.
//
// Tiles: 128 x 128 outputs per workgroup (4 waves, 64 x 64 each as 2 x 2
// MFMA blocks), K in steps of 32.  Both operand tiles go through LDS (rows
// padded to 80 B), double-buffered: the next K-tile's global loads are in
// flight in registers while the current one is multiplied, one barrier per
// K-tile.  At most 128 VGPRs and 40 KB of LDS per workgroup let four
// workgroups share a CU, so one waits on memory while the others multiply.
// Each output element is the same K-ordered sum whatever tile or chunk of
// rows it falls in, so results do not depend on how the rows are split.
#include "lsh_device.h"
#include "lsh_launch.h"

namespace lsh {

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kTS = 40;   // bf16 per staged row (32 + 8 pad: 80 B)

enum ALayout { kAF32Rows = 0, kABf16Rows = 1, kAF32Heads = 2, kABf16Heads = 3 };
constexpr bool a_bf16(int al) { return al == kABf16Rows || al == kABf16Heads; }
constexpr bool a_heads(int al) { return al == kAF32Heads || al == kABf16Heads; }
enum Epilogue { kEpiQkv = 0, kEpiResidual = 1, kEpiReluBf16 = 2 };

struct GemmArgs {
  const void* a;
  int64_t lda;          // rows layouts: element (m, k) at a[m * lda + k]
  int heads, L;         // heads layout: (m, k) at a[((m / L * heads + k / 64) * L + m % L) * 64 + k % 64]
  const uint16_t* w0;   // output features n < n0
  const uint16_t* w1;   // output features n >= n0 (row n - n0)
  int n0;
  int M, N, K;
  void* out0;           // qkv: qk; residual: out (fp32 [M][N]); relu: bf16 [M][N]
  void* out1;           // qkv: v
  const float* bias;    // [N] or null
  const float* resid;   // residual: fp32 [M][N] (may equal out0)
  float sign;           // residual: out = resid + sign * (acc + bias)
};

__device__ __forceinline__ uint32_t gemm_pack2(float a, float b) {
  const bf16x2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// One K-tile of A (128 rows x 32 k) in registers.
template <int AL>
struct GemmATile {
  uint4 r[a_bf16(AL) ? 2 : 4];
};

// Element offset of (row m, k = 0) of A for the rows this thread stages, or
// -1 past the last row.  Heads layout: k = 64h + j lies at
// ((b * H + h) * L + l) * 64 + j, i.e. row offset (b * H * L + l) * 64 plus
// h * L * 64 + j.
template <int AL>
struct GemmARows {
  int64_t off[a_bf16(AL) ? 2 : 4];
};

template <int AL>
__device__ __forceinline__ void gemm_a_rows(GemmARows<AL>& ar, const GemmArgs& g, int m0) {
#pragma unroll
  for (int q = 0; q < (a_bf16(AL) ? 2 : 4); ++q) {
    const int idx = threadIdx.x + 256 * q;
    const int m = m0 + (a_bf16(AL) ? idx >> 2 : idx >> 3);
    int64_t o = -1;
    if (m < g.M) {
      if (a_heads(AL)) {
        const int bi = m / g.L, l = m - bi * g.L;
        o = ((int64_t)bi * g.heads * g.L + l) * kHeadDim;
      } else {
        o = (int64_t)m * g.lda;
      }
    }
    ar.off[q] = o;
  }
}

// FULL: every row of the tile exists, so no load needs a guard (and the
// compiler needs no zero fill or branch per load).
template <int AL, bool FULL>
__device__ __forceinline__ void gemm_load_a(GemmATile<AL>& t, const GemmArgs& g,
                                            const GemmARows<AL>& ar, int k0) {
  if (a_bf16(AL)) {
    const uint16_t* a = static_cast<const uint16_t*>(g.a);
    // heads: the K-tile at k0 lies in head k0 / 64
    const int64_t kofs = AL == kABf16Heads
                             ? (int64_t)(k0 / kHeadDim) * g.L * kHeadDim + k0 % kHeadDim
                             : k0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c8 = ((threadIdx.x + 256 * q) & 3) * 8;
      t.r[q] = (FULL || ar.off[q] >= 0) ? load16(a + ar.off[q] + kofs + c8)
                                         : make_uint4(0, 0, 0, 0);
    }
  } else {
    const float* a = static_cast<const float*>(g.a);
    // heads: the K-tile at k0 lies in head k0 / 64
    const int64_t kofs = AL == kAF32Heads
                             ? (int64_t)(k0 / kHeadDim) * g.L * kHeadDim + k0 % kHeadDim
                             : k0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c4 = ((threadIdx.x + 256 * q) & 7) * 4;
      t.r[q] = (FULL || ar.off[q] >= 0) ? load16(a + ar.off[q] + kofs + c4)
                                         : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int AL>
__device__ __forceinline__ void gemm_store_a(uint16_t* as, const GemmATile<AL>& t) {
  if (a_bf16(AL)) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = threadIdx.x + 256 * q;
      store16(&as[(idx >> 2) * kTS + (idx & 3) * 8], t.r[q]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = threadIdx.x + 256 * q;
      const uint4 u = t.r[q];
      const uint2 p = make_uint2(gemm_pack2(__uint_as_float(u.x), __uint_as_float(u.y)),
                                 gemm_pack2(__uint_as_float(u.z), __uint_as_float(u.w)));
      *reinterpret_cast<uint2*>(&as[(idx >> 3) * kTS + (idx & 7) * 4]) = p;
    }
  }
}

template <bool FULL>
__device__ __forceinline__ void gemm_load_w(uint4 (&t)[2], const GemmArgs& g, int n_base, int k0) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = threadIdx.x + 256 * q;
    const int n = n_base + (idx >> 2), c8 = (idx & 3) * 8;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (FULL || n < g.N) {
      const uint16_t* row = n < g.n0 ? g.w0 + (int64_t)n * g.K : g.w1 + (int64_t)(n - g.n0) * g.K;
      u = load16(row + k0 + c8);
    }
    t[q] = u;
  }
}

__device__ __forceinline__ void gemm_store_w(uint16_t* ws, const uint4 (&t)[2]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = threadIdx.x + 256 * q;
    store16(&ws[(idx >> 2) * kTS + (idx & 3) * 8], t[q]);
  }
}

// The epilogue of one wave's 64 x 64 block, staged through the wave's own
// 9,216 bytes of the (by then idle) operand LDS so that every global access
// is a 16-byte piece of a full output row.  The products are taken as
// C^T = W A^T, so register r of lane l of block (i, j) holds feature
// 8*(r/4) + 4*(l/32) + r%4 of token l%32: registers 4q .. 4q+3 are four
// consecutive features of one token.  bf16 outputs (qk/v, the hidden layer)
// go through LDS in one pass of 64 rows x 128 B; fp32 outputs with the
// residual in two passes of 32 rows x 256 B.  The 64 features of a block
// are one head of qk or v (the block starts at a multiple of 64).
constexpr int kStageBf16 = 72;    // bf16 per staged row (128 B + 16 B pad)
constexpr int kStageF32 = 68;     // floats per staged row (256 B + 16 B pad)
static_assert(64 * kStageBf16 * 2 <= 9216 && 32 * kStageF32 * 4 <= 9216, "stage exceeds 9,216 B");
static_assert(2 * 9216 <= 2 * kBM * kTS * 2 && 2 * 9216 <= 2 * kBN * kTS * 2, "two stages per array");

template <int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, const f32x16 (&acc)[2][2], int mb,
                                              int nb, void* stage_mem) {
  const int lane = lane_id();
  if (EPI != kEpiResidual) {
    uint16_t* st = static_cast<uint16_t*>(stage_mem);
    float4 bias[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bias[j][q] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (EPI == kEpiReluBf16 && g.bias)
          bias[j][q] = *reinterpret_cast<const float4*>(
              g.bias + min(nb + j * 32 + 8 * q + 4 * (lane >> 5), g.N - 4));
      }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          if (EPI == kEpiReluBf16) {
            v[0] = fmaxf(v[0] + bias[j][q].x, 0.f);
            v[1] = fmaxf(v[1] + bias[j][q].y, 0.f);
            v[2] = fmaxf(v[2] + bias[j][q].z, 0.f);
            v[3] = fmaxf(v[3] + bias[j][q].w, 0.f);
          }
          const int row = i * 32 + (lane & 31), col = j * 32 + 8 * q + 4 * (lane >> 5);
          *reinterpret_cast<uint2*>(&st[row * kStageBf16 + col]) =
              make_uint2(gemm_pack2(v[0], v[1]), gemm_pack2(v[2], v[3]));
        }
    __builtin_amdgcn_wave_barrier();
    // 8 lanes per row, 16 bytes each: 8 rows per pass
    const int c8 = (lane & 7) * 8;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int row = p * 8 + (lane >> 3);
      const int m = mb + row;
      const uint4 u = *reinterpret_cast<const uint4*>(&st[row * kStageBf16 + c8]);
      if (m >= g.M || nb >= g.N) continue;
      if (EPI == kEpiQkv) {
        // features nb .. nb+63 of qk (nb < n0) or v: one head, [b][H][L][64]
        const int f = nb < g.n0 ? nb : nb - g.n0;
        uint16_t* out = static_cast<uint16_t*>(nb < g.n0 ? g.out0 : g.out1);
        const int bi = m / g.L, l = m - bi * g.L;
        store16(out + (((int64_t)bi * g.heads + f / kHeadDim) * g.L + l) * kHeadDim + c8, u);
      } else {
        store16(static_cast<uint16_t*>(g.out0) + (int64_t)m * g.N + nb + c8, u);
      }
    }
  } else {
    if (nb >= g.N) return;   // the block lies past the last feature (N % 128 == 64)
    float* st = static_cast<float*>(stage_mem);
    // 16 lanes per row, 16 bytes each: 4 rows per pass; a lane's columns
    // are the same in every pass
    const int c4 = (lane & 15) * 4;
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (g.bias) b = *reinterpret_cast<const float4*>(g.bias + nb + c4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = lane & 31, col = j * 32 + 8 * q + 4 * (lane >> 5);
          *reinterpret_cast<float4*>(&st[row * kStageF32 + col]) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]);
        }
      __builtin_amdgcn_wave_barrier();
      float4 rv[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int64_t mc = min(mb + i * 32 + p * 4 + (lane >> 4), g.M - 1);
        rv[p] = *reinterpret_cast<const float4*>(g.resid + mc * g.N + nb + c4);
      }
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int row = p * 4 + (lane >> 4);
        const int m = mb + i * 32 + row;
        const float4 a = *reinterpret_cast<const float4*>(&st[row * kStageF32 + c4]);
        if (m >= g.M) continue;
        const float v0 = a.x + b.x, v1 = a.y + b.y, v2 = a.z + b.z, v3 = a.w + b.w;
        *reinterpret_cast<float4*>(static_cast<float*>(g.out0) + (int64_t)m * g.N + nb + c4) =
            make_float4(rv[p].x + g.sign * v0, rv[p].y + g.sign * v1, rv[p].z + g.sign * v2,
                        rv[p].w + g.sign * v3);
      }
    }
  }
}

// The K loop: the next K-tile is requested while the current one is multiplied
// out of LDS (double-buffered), one barrier per K-tile.
template <int AL, bool FULL>
__device__ __forceinline__ void gemm_main_loop(const GemmArgs& g, const GemmARows<AL>& ar,
                                               int n_base, uint16_t (&as)[2][kBM * kTS],
                                               uint16_t (&ws)[2][kBN * kTS],
                                               f32x16 (&acc)[2][2]) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nkt = g.K / kBK;
  GemmATile<AL> ta;
  uint4 tw[2];
  gemm_load_a<AL, FULL>(ta, g, ar, 0);
  gemm_load_w<FULL>(tw, g, n_base, 0);
  gemm_store_a<AL>(as[0], ta);
  gemm_store_w(ws[0], tw);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) {   // next K-tile in flight during the products
      gemm_load_a<AL, FULL>(ta, g, ar, (kt + 1) * kBK);
      gemm_load_w<FULL>(tw, g, n_base, (kt + 1) * kBK);
    }
    const uint16_t* a_s = as[kt & 1];
    const uint16_t* w_s = ws[kt & 1];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kc = 16 * ks + 8 * (lane >> 5);
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = as_bf16x8(load16(&a_s[(wm * 64 + i * 32 + (lane & 31)) * kTS + kc]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = as_bf16x8(load16(&w_s[(wn * 64 + j * 32 + (lane & 31)) * kTS + kc]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      gemm_store_a<AL>(as[(kt + 1) & 1], ta);
      gemm_store_w(ws[(kt + 1) & 1], tw);
    }
    __syncthreads();
  }
}

// at most 128 VGPRs: four workgroups per CU hide each other's load latency
template <int AL, int EPI>
__global__ __launch_bounds__(256, 4) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t as[2][kBM * kTS];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kBN * kTS];
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int ntn = (g.N + kBN - 1) / kBN;
  // each XCD takes a contiguous range of row tiles, so its A rows stay in its L2
  const int64_t blk = xcd_logical_block(blockIdx.x, gridDim.x);
  const int m0 = (int)(blk / ntn) * kBM;
  const int n_base = (int)(blk % ntn) * kBN;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  GemmARows<AL> ar;
  gemm_a_rows<AL>(ar, g, m0);
  // the usual case: the whole tile lies inside M and N
  if (m0 + kBM <= g.M && n_base + kBN <= g.N)
    gemm_main_loop<AL, true>(g, ar, n_base, as, ws, acc);
  else
    gemm_main_loop<AL, false>(g, ar, n_base, as, ws, acc);

  // every wave is past its last operand reads (the loop ends on a barrier):
  // waves 0-1 stage their outputs in as, waves 2-3 in ws
  char* stage = wave < 2 ? reinterpret_cast<char*>(&as[0][0]) + wave * 9216
                         : reinterpret_cast<char*>(&ws[0][0]) + (wave - 2) * 9216;
  gemm_epilogue<EPI>(g, acc, m0 + wm * 64, n_base + wn * 64, stage);
}

template <int AL, int EPI>
hipError_t gemm_launch(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = (int64_t)((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<AL, EPI>), dim3((unsigned)tiles), dim3(256), 0, stream, g);
  return hipGetLastError();
}

static GemmArgs gemm_args(int M, int N, int K) {
  GemmArgs g = {};
  g.M = M;
  g.N = N;
  g.K = K;
  g.n0 = N;
  g.sign = 1.f;
  return g;
}

hipError_t launch_project_qkv(const LayerShape& s, const float* x, const uint16_t* w_qk,
                              const uint16_t* w_v, uint16_t* qk, uint16_t* v,
                              hipStream_t stream) {
  GemmArgs g = gemm_args(s.batch * s.len, 2 * s.d_model, s.d_model);
  g.a = x;
  g.lda = s.d_model;
  g.heads = s.d_model / kHeadDim;
  g.L = s.len;
  g.w0 = w_qk;
  g.w1 = w_v;
  g.n0 = s.d_model;
  g.out0 = qk;
  g.out1 = v;
  return gemm_launch<kAF32Rows, kEpiQkv>(g, stream);
}

hipError_t launch_project_out(const LayerShape& s, const float* y_att, const uint16_t* w_o,
                              const float* resid, float sign, float* out, hipStream_t stream) {
  GemmArgs g = gemm_args(s.batch * s.len, s.d_model, s.d_model);
  g.a = y_att;
  g.heads = s.d_model / kHeadDim;
  g.L = s.len;
  g.w0 = g.w1 = w_o;
  g.out0 = out;
  g.resid = resid;
  g.sign = sign;
  return gemm_launch<kAF32Heads, kEpiResidual>(g, stream);
}

hipError_t launch_project_out_bf16(const LayerShape& s, const uint16_t* y_att,
                                   const uint16_t* w_o, const float* resid, float sign,
                                   float* out, hipStream_t stream) {
  GemmArgs g = gemm_args(s.batch * s.len, s.d_model, s.d_model);
  g.a = y_att;
  g.heads = s.d_model / kHeadDim;
  g.L = s.len;
  g.w0 = g.w1 = w_o;
  g.out0 = out;
  g.resid = resid;
  g.sign = sign;
  return gemm_launch<kABf16Heads, kEpiResidual>(g, stream);
}

hipError_t launch_ffn(const LayerShape& s, const float* x, const uint16_t* w_1, const float* b_1,
                      const uint16_t* w_2, const float* b_2, const float* resid, float sign,
                      float* out, uint16_t* hidden, hipStream_t stream) {
  const int64_t rows = (int64_t)s.batch * s.len;
  const int64_t chunk = s.ffn_chunk > 0 ? s.ffn_chunk : rows;
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    const int m = (int)(rows - r0 < chunk ? rows - r0 : chunk);
    // hidden = bf16(ReLU(x W1^T + b1)) for this chunk of tokens
    GemmArgs g1 = gemm_args(m, s.d_ff, s.d_model);
    g1.a = x + r0 * s.d_model;
    g1.lda = s.d_model;
    g1.w0 = g1.w1 = w_1;
    g1.bias = b_1;
    g1.out0 = hidden;
    hipError_t e = gemm_launch<kAF32Rows, kEpiReluBf16>(g1, stream);
    if (e != hipSuccess) return e;
    // out = resid + sign * (hidden W2^T + b2)
    GemmArgs g2 = gemm_args(m, s.d_model, s.d_ff);
    g2.a = hidden;
    g2.lda = s.d_ff;
    g2.w0 = g2.w1 = w_2;
    g2.bias = b_2;
    g2.out0 = out + r0 * s.d_model;
    g2.resid = resid + r0 * s.d_model;
    g2.sign = sign;
    e = gemm_launch<kABf16Rows, kEpiResidual>(g2, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lsh
