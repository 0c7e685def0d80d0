// MFMA (bf16 in, fp32 accumulate) kernels of the Hutchinson estimator on
// gfx950 (the randomized-clipping summary, section 中核メカニズム, item 1):
//   sketch   Y_i = G_i P_i      reduction along each token row (contiguous)
//   project  Z_i = A_i^T Y_i    reduction along the tokens (strided rows)
// Both stream their big operand from HBM exactly once with 16-byte loads and
// feed v_mfma_f32_16x16x32_bf16 directly from registers.
//
// MFMA operand facts used (16x16x32 bf16, wave64): lane l supplies row l % 16
// of A and column l % 16 of B, each with 8 bf16 of the contraction index; the
// result D[4 (l / 16) + i][l % 16] sits in accumulator register i of lane l.
// Which 8 contraction indices a lane group holds is free, as long as the A and
// B operands agree; the kernels use that freedom to make every lane's 8 values
// one contiguous 16-byte load.
#include "common.h"
#include "internal.h"

namespace dprc {

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const bf16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ---------------------------------------------------------------------------
// Sketch.  A workgroup (NW waves) owns 16*MB tokens of one sample; wave w
// reduces the slice r in [w W/NW, (w+1) W/NW) in steps of 64.  In a step, lane
// (m = l % 16, g = l / 16) loads 32 contiguous bytes of token row m at offset
// 16 g; contraction slot (h, g, e) is r = r0 + 16 g + 8 h + e for both the
// token rows (A operand) and the probe rows P^T[j] (B operand).  The waves'
// partial Y tiles are summed in LDS in a fixed order and stored as bf16
// Y^T[b][j][t].  Every workgroup re-reads its sample's probe rows (32 x W)
// from L2: 64-token workgroups read half a byte of P per byte of X, 128-token
// ones a quarter, which is what wide rows (W >= 4096) need; narrower rows keep
// 64 tokens and four waves, whose loops would otherwise be too short.
// ---------------------------------------------------------------------------
constexpr int kSketchK = 64;

// The workgroup of token block tb of sample b.
template <int MB, int NW>
__device__ __forceinline__ void sketch_body(const bf16_t* __restrict__ X, int T, int W,
                                            const bf16_t* __restrict__ P, int64_t p_bstride,
                                            bf16_t* __restrict__ Y, int tb, int b) {
  constexpr int TM = 16 * MB;
  __shared__ float red[NW][32][TM + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int t0 = tb * TM;
  const int Wq = W / NW;
  const int rbeg = wave * Wq + 16 * g;

  const bf16_t* xr[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    xr[mb] = X + (static_cast<int64_t>(b) * T + t0 + mb * 16 + m) * W + rbeg;
  const bf16_t* pr[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
    pr[nb] = P + b * p_bstride + static_cast<int64_t>(nb * 16 + m) * W + rbeg;

  f32x4 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xa[2][MB][2], pv[2][2][2];
  auto load = [&](int buf, int r) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int h = 0; h < 2; ++h) xa[buf][mb][h] = ld16(xr[mb] + r + 8 * h);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h) pv[buf][nb][h] = ld16(pr[nb] + r + 8 * h);
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma16(xa[buf][mb][h], pv[buf][nb][h], acc[mb][nb]);
  };

  const int niter = Wq / kSketchK;
  load(0, 0);
  for (int it = 0; it < niter; it += 2) {
    if (it + 1 < niter) load(1, (it + 1) * kSketchK);
    compute(0);
    if (it + 1 < niter) {
      if (it + 2 < niter) load(0, (it + 2) * kSketchK);
      compute(1);
    }
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][nb * 16 + m][mb * 16 + 4 * g + i] = acc[mb][nb][i];
  __syncthreads();

  // 32 x TM outputs over the first 256 threads, TM / 8 consecutive tokens each.
  constexpr int PER = TM / 8;
  if (threadIdx.x >= 256) return;
  const int j = threadIdx.x >> 3;
  const int tc = (threadIdx.x & 7) * PER;
  uint32_t packed[PER / 2];
#pragma unroll
  for (int u = 0; u < PER; u += 2) {
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      v0 += red[w][j][tc + u];
      v1 += red[w][j][tc + u + 1];
    }
    packed[u / 2] = pack_bf16x2(v0, v1);
  }
  bf16_t* dst = Y + (static_cast<int64_t>(b) * kMfmaProbeCols + j) * T + t0 + tc;
  if constexpr (PER >= 8) {
#pragma unroll
    for (int c = 0; c < PER / 8; ++c) {
      u32x4 v{packed[4 * c], packed[4 * c + 1], packed[4 * c + 2], packed[4 * c + 3]};
      *reinterpret_cast<u32x4*>(dst + 8 * c) = v;
    }
  } else {
    uint2 v{packed[0], packed[1]};
    *reinterpret_cast<uint2*>(dst) = v;
  }
}

template <int MB, int NW>
__global__ void __launch_bounds__(64 * NW) k_sketch_mfma(const bf16_t* __restrict__ X, int T, int W,
                                                     const bf16_t* __restrict__ P,
                                                     int64_t p_bstride, bf16_t* __restrict__ Y) {
  sketch_body<MB, NW>(X, T, W, P, p_bstride, Y, blockIdx.x, blockIdx.y);
}

// Several layers of one shape class in one launch: layer blockIdx.z of the table.
template <int MB, int NW>
__global__ void __launch_bounds__(64 * NW) k_sketch_mfma_layers(int T, SketchLayers tab) {
  const int l = blockIdx.z;
  sketch_body<MB, NW>(tab.X[l], T, tab.W[l], tab.P[l], tab.pbs[l], tab.Y[l], blockIdx.x,
                      blockIdx.y);
}

bool mfma_sketch_ok(int T, int W) { return T > 0 && T % 32 == 0 && W % (4 * kSketchK) == 0; }

// Sketch shape: 2 = 128-token workgroups of 8 waves (rows of 4096+ features),
// 1 = 64 tokens and 4 waves, 0 = 32 tokens and 4 waves (few token blocks).
int mfma_sketch_variant(int B, int T, int W) {
  if (T % 128 == 0 && W >= 4096 && W % (8 * kSketchK) == 0 &&
      static_cast<int64_t>(B) * (T / 128) >= 256)
    return 2;
  if (T % 64 == 0 && static_cast<int64_t>(B) * (T / 64) >= 512) return 1;
  return 0;
}

hipError_t launch_sketch_mfma(const bf16_t* X, int B, int T, int W, const bf16_t* P,
                              int64_t p_bstride, bf16_t* Y, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!mfma_sketch_ok(T, W)) return hipErrorInvalidValue;
  switch (mfma_sketch_variant(B, T, W)) {
    case 2:
      hipLaunchKernelGGL((k_sketch_mfma<8, 8>), dim3(T / 128, B), dim3(512), 0, s, X, T, W, P,
                         p_bstride, Y);
      break;
    case 1:
      hipLaunchKernelGGL((k_sketch_mfma<4, 4>), dim3(T / 64, B), dim3(256), 0, s, X, T, W, P,
                         p_bstride, Y);
      break;
    default:
      hipLaunchKernelGGL((k_sketch_mfma<2, 4>), dim3(T / 32, B), dim3(256), 0, s, X, T, W, P,
                         p_bstride, Y);
  }
  return hipGetLastError();
}

hipError_t launch_sketch_mfma_layers(int variant, int B, int T, const SketchLayers& tab,
                                     hipStream_t s) {
  if (B <= 0 || tab.n <= 0) return hipSuccess;
  if (tab.n > kNormLayersMax) return hipErrorInvalidValue;
  for (int l = 0; l < tab.n; ++l)
    if (!mfma_sketch_ok(T, tab.W[l]) || mfma_sketch_variant(B, T, tab.W[l]) != variant)
      return hipErrorInvalidValue;
  switch (variant) {
    case 2:
      hipLaunchKernelGGL((k_sketch_mfma_layers<8, 8>), dim3(T / 128, B, tab.n), dim3(512), 0, s, T,
                         tab);
      break;
    case 1:
      hipLaunchKernelGGL((k_sketch_mfma_layers<4, 4>), dim3(T / 64, B, tab.n), dim3(256), 0, s, T,
                         tab);
      break;
    default:
      hipLaunchKernelGGL((k_sketch_mfma_layers<2, 4>), dim3(T / 32, B, tab.n), dim3(256), 0, s, T,
                         tab);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Project.  A workgroup owns 16 CW columns q of one sample (CW = 8: 128
// columns, CW = 4: 64) and one token split; wave w takes a contiguous quarter
// of the split in steps of 32 tokens.  In a step, lane (m, g) loads tokens
// t0 + 8 g + e (e = 0..7) of the CW-column group q0 + CW m (16 or 8 bytes);
// an in-register transpose of those 16-bit values gives the A operand of CW
// MFMA blocks, block c holding rows q = q0 + CW m + c.  The B operand is
// Y^T[j][t0 + 8 g .. + 7], one 16-byte load.  Contraction slot (g, e) is token
// t0 + 8 g + e for both operands.
//
// SQ = false: the workgroup's 32 x 16 CW tile of Z (one split) is stored to
// the fp32 partials Zp[b][split].  SQ = true (one split, so the tile is final):
// the workgroup reduces it at once to sum_j w_j sum_q Z[j][q]^2 in fp64 (the
// weighted squared Frobenius norm restricted to its columns; w_j = w0 for
// j < n0, w1 for the next n1, 0 for padding) and stores that one double to
// part[b][column block], so no Z partials are written or read back.
// ---------------------------------------------------------------------------
constexpr int kProjK = 32;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int CW> struct ProjRow;
template <> struct ProjRow<8> { typedef u32x4 type; };
template <> struct ProjRow<4> { typedef u32x2 type; };

// Column c of eight rows of 16-bit values (rows[e] holds 2 per dword), as the
// MFMA's 8 contraction values (4 dwords, row e in slot e).
template <typename R>
__device__ __forceinline__ u32x4 transpose_col(const R* rows, int c) {
  u32x4 a;
  const int w = c >> 1;
  if ((c & 1) == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = (rows[2 * k][w] & 0xFFFFu) | (rows[2 * k + 1][w] << 16);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = (rows[2 * k][w] >> 16) | (rows[2 * k + 1][w] & 0xFFFF0000u);
  }
  return a;
}

// The workgroup of column block qb, token split `split`, sample b.
template <int CW, bool SQ>
__device__ __forceinline__ void project_body(const bf16_t* __restrict__ X, int T, int W,
                                             const bf16_t* __restrict__ Y, int split_tokens,
                                             int nsplit, float* __restrict__ Zp, int n0, float w0,
                                             int n1, float w1, double* __restrict__ part,
                                             int64_t part_stride, int qb, int split, int b) {
  constexpr int kQ = 16 * CW;
  typedef typename ProjRow<CW>::type RowT;
  __shared__ float red[4][32][kQ + 4];
  __shared__ double dred[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int q0 = qb * kQ;
  const int tw = split_tokens >> 2;
  const int tbeg = split * split_tokens + wave * tw;

  const bf16_t* xbase = X + (static_cast<int64_t>(b) * T + tbeg + 8 * g) * W + q0 + CW * m;
  const bf16_t* yb0 = Y + (static_cast<int64_t>(b) * kMfmaProbeCols + m) * T + tbeg + 8 * g;
  const bf16_t* yb1 = yb0 + static_cast<int64_t>(16) * T;

  f32x4 acc[CW][2];
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    acc[c][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // An iteration covers U = 8 / CW sub-steps of 32 tokens (sub-step u: tokens
  // t + 32 u + 8 g + e), so that a lane has 128 bytes of X in flight per buffer
  // whatever the column block.
  constexpr int U = 8 / CW;
  RowT rows[2][8 * U];
  u32x4 yv[2][U][2];
  auto load = [&](int buf, int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        rows[buf][8 * u + e] =
            *reinterpret_cast<const RowT*>(xbase + static_cast<int64_t>(t + kProjK * u + e) * W);
      yv[buf][u][0] = ld16(yb0 + t + kProjK * u);
      yv[buf][u][1] = ld16(yb1 + t + kProjK * u);
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        const u32x4 a = transpose_col(&rows[buf][8 * u], c);
        acc[c][0] = mfma16(a, yv[buf][u][0], acc[c][0]);
        acc[c][1] = mfma16(a, yv[buf][u][1], acc[c][1]);
      }
  };

  const int niter = tw / (kProjK * U);
  load(0, 0);
  for (int it = 0; it < niter; it += 2) {
    if (it + 1 < niter) load(1, (it + 1) * kProjK * U);
    compute(0);
    if (it + 1 < niter) {
      if (it + 2 < niter) load(0, (it + 2) * kProjK * U);
      compute(1);
    }
  }

  // D[row][col] of block (c, nb) sits in lane (col, g), register i, row 4 g + i:
  // probe j = 16 nb + col, column q0 + CW (4 g + i) + c.
#pragma unroll
  for (int c = 0; c < CW; ++c)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][nb * 16 + m][CW * (4 * g + i) + c] = acc[c][nb][i];
  __syncthreads();

  // 32 x kQ outputs: thread -> row j = tid / 8, kQ / 8 consecutive q.
  constexpr int PER = kQ / 8;
  const int j = threadIdx.x >> 3;
  const int qc = (threadIdx.x & 7) * PER;
  if constexpr (SQ) {
    const float w = j < n0 ? w0 : (j < n0 + n1 ? w1 : 0.f);
    double sq = 0.0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const float z = red[0][j][qc + u] + red[1][j][qc + u] + red[2][j][qc + u] + red[3][j][qc + u];
      sq += static_cast<double>(z) * z;
    }
    const double tot = block_sum_d(static_cast<double>(w) * sq, dred);
    if (threadIdx.x == 0) part[static_cast<int64_t>(b) * part_stride + qb] = tot;
  } else {
    float* dst = Zp + ((static_cast<int64_t>(b) * nsplit + split) * kMfmaProbeCols + j) * W + q0 + qc;
#pragma unroll
    for (int u = 0; u < PER; u += 4) {
      float4 v;
      v.x = red[0][j][qc + u + 0] + red[1][j][qc + u + 0] + red[2][j][qc + u + 0] + red[3][j][qc + u + 0];
      v.y = red[0][j][qc + u + 1] + red[1][j][qc + u + 1] + red[2][j][qc + u + 1] + red[3][j][qc + u + 1];
      v.z = red[0][j][qc + u + 2] + red[1][j][qc + u + 2] + red[2][j][qc + u + 2] + red[3][j][qc + u + 2];
      v.w = red[0][j][qc + u + 3] + red[1][j][qc + u + 3] + red[2][j][qc + u + 3] + red[3][j][qc + u + 3];
      *reinterpret_cast<float4*>(dst + u) = v;
    }
  }
}

template <int CW, bool SQ>
__global__ void __launch_bounds__(256) k_project_mfma(const bf16_t* __restrict__ X, int T, int W,
                                                      const bf16_t* __restrict__ Y,
                                                      int split_tokens, int nsplit,
                                                      float* __restrict__ Zp, int n0, float w0,
                                                      int n1, float w1,
                                                      double* __restrict__ part,
                                                      int64_t part_stride) {
  project_body<CW, SQ>(X, T, W, Y, split_tokens, nsplit, Zp, n0, w0, n1, w1, part, part_stride,
                       blockIdx.x, blockIdx.y, blockIdx.z);
}

// The fused projection-and-square of several layers in one launch: layer
// blockIdx.y of the table, its column blocks blockIdx.x < W / (16 CW).
template <int CW>
__global__ void __launch_bounds__(256) k_project_sq_layers(int T, ProjectLayers tab, int n0,
                                                           float w0, int n1, float w1,
                                                           double* __restrict__ part,
                                                           int64_t part_stride) {
  const int l = blockIdx.y;
  const int W = tab.W[l];
  if (static_cast<int>(blockIdx.x) >= W / (16 * CW)) return;
  project_body<CW, true>(tab.X[l], T, W, tab.Y[l], T, 1, nullptr, n0, w0, n1, w1,
                         part + tab.pbase[l], part_stride, blockIdx.x, 0, blockIdx.z);
}

// ---------------------------------------------------------------------------
// Finish (randomized-clipping summary, section 中核メカニズム, item 1: the
// estimate is the weighted squared Frobenius norm of Z = sum of the token
// splits), in two fixed-order passes.  Block (c, b) takes the float4
// positions 512 c .. 512 c + 511 of sample b's [32][W] rows, two per thread
// with every split's loads in flight, sums the splits in order and the
// weighted squares in fp64, and writes one partial; k_sum_parts then adds the
// sample's W / 64 partials in block order.  There are enough blocks to stream
// the splits at any B (one block per sample left two CUs at work at B = 2).
// Positions past the end load the last element (in bounds) and count zero, so
// no load sits under a branch.  No block communicates with another, so no
// atomics or fences are needed and the result is deterministic.
// ---------------------------------------------------------------------------
constexpr int kFrobThreads = 256, kFrobU = 2;

int mfma_frob_chunks(int W) {
  const int E4 = kMfmaProbeCols * W / 4;
  return (E4 + kFrobThreads * kFrobU - 1) / (kFrobThreads * kFrobU);
}

__global__ void __launch_bounds__(kFrobThreads) k_frob_chunks(const float* __restrict__ Zp,
                                                              int nsplit, int W, int n0, float w0,
                                                              int n1, float w1,
                                                              double* __restrict__ part,
                                                              int nchunk) {
  __shared__ double red[16];
  const int c = blockIdx.x, b = blockIdx.y;
  const int E4 = kMfmaProbeCols * W / 4;
  const float4* zb = reinterpret_cast<const float4*>(Zp) + static_cast<int64_t>(b) * nsplit * E4;
  const int u0 = c * kFrobThreads * kFrobU + threadIdx.x;
  int uc[kFrobU];
  float4 z[kFrobU];
#pragma unroll
  for (int q = 0; q < kFrobU; ++q) {
    const int u = u0 + kFrobThreads * q;
    uc[q] = u < E4 ? u : E4 - 1;
    z[q] = zb[uc[q]];
  }
#pragma unroll 4
  for (int sp = 1; sp < nsplit; ++sp) {
    float4 v[kFrobU];
#pragma unroll
    for (int q = 0; q < kFrobU; ++q) v[q] = zb[static_cast<int64_t>(sp) * E4 + uc[q]];
#pragma unroll
    for (int q = 0; q < kFrobU; ++q) {
      z[q].x += v[q].x;
      z[q].y += v[q].y;
      z[q].z += v[q].z;
      z[q].w += v[q].w;
    }
  }
  double acc = 0.0;
#pragma unroll
  for (int q = 0; q < kFrobU; ++q) {
    const int u = u0 + kFrobThreads * q;
    const int j = (4 * u) / W;  // probe column of this float4 (W % 4 == 0)
    const float w = j < n0 ? w0 : (j < n0 + n1 ? w1 : 0.f);
    if (u < E4 && w != 0.f)
      acc += static_cast<double>(w) *
             (static_cast<double>(z[q].x) * z[q].x + static_cast<double>(z[q].y) * z[q].y +
              static_cast<double>(z[q].z) * z[q].z + static_cast<double>(z[q].w) * z[q].w);
  }
  acc = block_sum_d(acc, red);
  if (threadIdx.x == 0) part[static_cast<int64_t>(b) * nchunk + c] = acc;
}

hipError_t launch_frob_finish(const float* Zp, int B, int nsplit, int W, int n0, float w0, int n1,
                              float w1, double* part, float* n_sq, int accumulate, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (W % 4 != 0 || nsplit < 1) return hipErrorInvalidValue;
  const int nchunk = mfma_frob_chunks(W);
  hipLaunchKernelGGL(k_frob_chunks, dim3(nchunk, B), dim3(kFrobThreads), 0, s, Zp, nsplit, W, n0,
                     w0, n1, w1, part, nchunk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_parts(part, B, nchunk, n_sq, accumulate, s);
}

hipError_t launch_project_sq_mfma_layers(int B, int T, int cols, const ProjectLayers& tab, int n0,
                                         float w0, int n1, float w1, double* part,
                                         int64_t part_stride, hipStream_t s) {
  if (B <= 0 || tab.n <= 0) return hipSuccess;
  if (tab.n > kNormLayersMax || (cols != 64 && cols != 128)) return hipErrorInvalidValue;
  int maxblk = 0;
  for (int l = 0; l < tab.n; ++l) {
    if (mfma_project_sq_cols(B, T, tab.W[l]) != cols) return hipErrorInvalidValue;
    maxblk = tab.W[l] / cols > maxblk ? tab.W[l] / cols : maxblk;
  }
  if (cols == 128) {
    hipLaunchKernelGGL((k_project_sq_layers<8>), dim3(maxblk, tab.n, B), dim3(256), 0, s, T, tab, n0,
                       w0, n1, w1, part, part_stride);
  } else {
    hipLaunchKernelGGL((k_project_sq_layers<4>), dim3(maxblk, tab.n, B), dim3(256), 0, s, T, tab, n0,
                       w0, n1, w1, part, part_stride);
  }
  return hipGetLastError();
}

bool mfma_project_ok(int T, int W) { return T > 0 && T % (4 * kProjK) == 0 && W % 128 == 0; }

// Token splits of the 128-column projection: about 256 workgroups in all
// (fewer splits mean fewer fp32 partials to write and re-read; measured
// best), each split a multiple of 128 tokens dividing T.
int mfma_project_splits(int B, int T, int W) {
  const int64_t base = static_cast<int64_t>(B) * (W / 128);
  int want = static_cast<int>((256 + base - 1) / (base > 0 ? base : 1));
  const int maxs = T / (4 * kProjK);
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  for (int s = want; s >= 1; --s)
    if (T % (s * 4 * kProjK) == 0) return s;
  return 1;
}

hipError_t launch_project_mfma(const bf16_t* X, int B, int T, int W, const bf16_t* Y, int nsplit,
                               float* Zp, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!mfma_project_ok(T, W) || nsplit < 1 || T % (nsplit * 4 * kProjK) != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_project_mfma<8, false>), dim3(W / 128, nsplit, B), dim3(256), 0, s, X, T,
                     W, Y, T / nsplit, nsplit, Zp, 0, 0.f, 0, 0.f, nullptr, 0);
  return hipGetLastError();
}

// Column block of the fused projection-and-square: 128 columns when that
// alone gives at least 256 workgroups, else 64 when that does; 0 when neither
// does (the caller then takes the split projection and the finish).
int mfma_project_sq_cols(int B, int T, int W) {
  if (B <= 0 || !mfma_project_ok(T, W)) return 0;
  const int64_t b = B;
  if (b * (W / 128) >= 256) return 128;
  if (b * (W / 64) >= 256 && T % (4 * 2 * kProjK) == 0) return 64;
  return 0;
}

hipError_t launch_project_sq_mfma(const bf16_t* X, int B, int T, int W, const bf16_t* Y, int cols,
                                  int n0, float w0, int n1, float w1, double* part,
                                  int64_t part_stride, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!mfma_project_ok(T, W) || (cols != 64 && cols != 128) || (cols == 64 && T % 256 != 0))
    return hipErrorInvalidValue;
  if (cols == 128) {
    hipLaunchKernelGGL((k_project_mfma<8, true>), dim3(W / 128, 1, B), dim3(256), 0, s, X, T, W, Y,
                       T, 1, nullptr, n0, w0, n1, w1, part, part_stride);
  } else {
    hipLaunchKernelGGL((k_project_mfma<4, true>), dim3(W / 64, 1, B), dim3(256), 0, s, X, T, W, Y,
                       T, 1, nullptr, n0, w0, n1, w1, part, part_stride);
  }
  return hipGetLastError();
}

}  // namespace dprc
