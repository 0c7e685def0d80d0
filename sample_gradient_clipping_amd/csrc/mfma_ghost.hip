// Ghost-clipping baseline on MFMA (bf16 in, fp32 accumulate), gfx950.
//
//   n_i = sum_{s,t} (A_i A_i^T)_{st} (G_i G_i^T)_{st}
//
// (randomized-clipping summary, sections 問題定義 and 1. 複雑性の削減: ghost
// clipping works with T x T Gram products, O(T^2 (p + d)) work per sample; the
// trace identity of section 中核メカニズム makes it equal to ||A_i^T G_i||_F^2.)
//
// One workgroup per (sample, pair of 128-token blocks sb <= tb).  It forms the
// 128 x 128 tile of A A^T over the d features, then the same tile of G G^T over
// the p features, multiplies them elementwise and sums; off-diagonal tile pairs
// count twice (the Grams are symmetric), so only the upper triangle of tiles
// is computed.  Both Gram operands are token rows with the contraction index
// (features) contiguous, which is the MFMA operand layout as stored: 64-feature
// slabs of the two token blocks are staged in LDS and read with 16-byte reads.
// Four waves of 64 x 64 (2 x 2 blocks of v_mfma_f32_32x32x16_bf16) per tile.
// The tile pairs are dealt to the eight XCDs in contiguous runs of an order
// that walks 8 x 8 super-tiles of token blocks, so that the 64 workgroups an
// XCD holds at a time share 16 token blocks in its L2.
#include "common.h"
#include "internal.h"

namespace dprc {

constexpr int kTB = 128;             // tokens per block
constexpr int kKC = 64;              // features per LDS slab
constexpr int kRowB = kKC * 2 + 16;  // padded LDS row: 64 bf16 + 16 B
constexpr int kSlabBytes = 2 * kTB * kRowB;

__device__ __forceinline__ f32x16 mfma32g(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One Gram tile G_tile = X[s-block] X[t-block]^T over K features into acc
// (per wave 64 x 64 as 2 x 2 blocks of 32 x 32).
__device__ __forceinline__ void gram_tile(const bf16_t* __restrict__ xs,
                                          const bf16_t* __restrict__ xt, int K,
                                          unsigned char* lds, f32x16 (&acc)[2][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ws = wave >> 1, wt = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // staging: unit u = tid + 256 i covers side u / 1024, row (u % 1024) / 8,
  // 16-byte chunk u % 8 of the slab.
  u32x4 st[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = tid + 256 * i;
      const int side = u >> 10, row = (u & 1023) >> 3, ch = u & 7;
      const bf16_t* src = (side == 0 ? xs : xt) + static_cast<int64_t>(row) * K + k0 + ch * 8;
      st[i] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = tid + 256 * i;
      const int side = u >> 10, row = (u & 1023) >> 3, ch = u & 7;
      *reinterpret_cast<u32x4*>(lds + side * kTB * kRowB + row * kRowB + ch * 16) = st[i];
    }
  };
  // operand reads: lane (m = l % 32, g = l / 32) takes row m of a 32-row block,
  // features 16 ks + 8 g .. + 7.
  const int m = lane & 31, g = lane >> 5;
  const unsigned char* ra = lds + (ws * 64 + m) * kRowB + g * 16;
  const unsigned char* rb = lds + kTB * kRowB + (wt * 64 + m) * kRowB + g * 16;
  gload(0);
  for (int k0 = 0; k0 < K; k0 += kKC) {
    __syncthreads();  // previous slab consumed
    lstore();
    __syncthreads();
    if (k0 + kKC < K) gload(k0 + kKC);
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      u32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const u32x4*>(ra + i * 32 * kRowB + ks * 32);
        b[i] = *reinterpret_cast<const u32x4*>(rb + i * 32 * kRowB + ks * 32);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32g(a[i], b[j], acc[i][j]);
    }
  }
}

// Upper-triangle pair index -> token blocks (sb, tb), sb <= tb.  With nb a
// multiple of 8 the pairs are ordered in 8 x 8 super-tiles (I <= J, row by
// row; a diagonal super-tile holds its 36 pairs a <= c), so that a run of 64
// consecutive pairs needs only 16 token blocks; otherwise row by row.
__device__ __forceinline__ void pair_blocks(int pair, int nb, int& sb, int& tb) {
  int rem = pair;
  if (nb % 8 == 0) {
    const int nsup = nb / 8;
    int I = 0, J = 0;
    for (;;) {
      const int size = I == J ? 36 : 64;
      if (rem < size) break;
      rem -= size;
      if (++J == nsup) {
        ++I;
        J = I;
      }
    }
    int a, c;
    if (I == J) {
      a = 0;
      while (rem >= 8 - a) {
        rem -= 8 - a;
        ++a;
      }
      c = a + rem;
    } else {
      a = rem >> 3;
      c = rem & 7;
    }
    sb = 8 * I + a;
    tb = 8 * J + c;
    return;
  }
  sb = 0;
  while (rem >= nb - sb) {
    rem -= nb - sb;
    ++sb;
  }
  tb = sb + rem;
}

__global__ void __launch_bounds__(256) k_ghost_mfma(const bf16_t* __restrict__ A,
                                                    const bf16_t* __restrict__ G, int T, int d,
                                                    int p, double* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kSlabBytes];
  __shared__ double red[4];
  const int b = blockIdx.y;
  const int nb = T / kTB;
  const int npair = gridDim.x;
  const int w = blockIdx.x;  // consecutive workgroups go to the eight XCDs in turn
  const int pair = (npair % 8 == 0) ? (w % 8) * (npair / 8) + w / 8 : w;
  int sb, tb;
  pair_blocks(pair, nb, sb, tb);
  const bf16_t* as = A + (static_cast<int64_t>(b) * T + sb * kTB) * d;
  const bf16_t* at = A + (static_cast<int64_t>(b) * T + tb * kTB) * d;
  const bf16_t* gs = G + (static_cast<int64_t>(b) * T + sb * kTB) * p;
  const bf16_t* gt = G + (static_cast<int64_t>(b) * T + tb * kTB) * p;
  f32x16 ga[2][2], gg[2][2];
  gram_tile(as, at, d, lds, ga);
  gram_tile(gs, gt, p, lds, gg);
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        acc += static_cast<double>(ga[i][j][e]) * static_cast<double>(gg[i][j][e]);
  acc = wave_sum_d(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double w = sb == tb ? 1.0 : 2.0;
    part[static_cast<int64_t>(b) * gridDim.x + pair] = w * (red[0] + red[1] + red[2] + red[3]);
  }
}

bool mfma_ghost_ok(int T, int d, int p) {
  return T > 0 && T % kTB == 0 && d % kKC == 0 && p % kKC == 0;
}

int mfma_ghost_nparts(int T) {
  const int nb = T / kTB;
  return nb * (nb + 1) / 2;
}

hipError_t launch_ghost_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p,
                             double* part, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!mfma_ghost_ok(T, d, p)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_ghost_mfma, dim3(mfma_ghost_nparts(T), B), dim3(256), 0, s, A, G, T, d, p,
                     part);
  return hipGetLastError();
}

}  // namespace dprc
