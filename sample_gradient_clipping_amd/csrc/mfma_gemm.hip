// MFMA contraction over tokens for bf16 inputs on gfx950:
//   aggregate   part[split][o][q] = sum_{tokens} c_i G_i[t][o] A_i[t][q]
//               (the clipped sum S = sum_i c_i G_i^T A_i: glossary page, section
//               DP-SGDのアルゴリズム, step 4; randomized-clipping summary,
//               section アルゴリズム的フロー, step 5)
//   fgc         M_i[o][q]            = sum_t G_i[t][o] A_i[t][q]   (FGC baseline)
// M = o (p), N = q (d), K = tokens.  Both operands are stored token-major, so
// the contraction index is the strided one: each 8 x 8 block of 16-bit values
// is transposed in registers on its way into LDS, where every column then
// holds its 64 tokens contiguously and MFMA operands are single 16-byte reads.
//
// Workgroup tile 256 x 256, four waves of 128 x 128 (8 x 8 blocks of
// v_mfma_f32_16x16x32_bf16), 32 tokens per stage, two LDS stages.
//
// Per-sample clip factors without a second accumulator: the active samples are
// visited in ascending c, and the accumulator holds sum_{seen} (c_seg / c_cur)
// S_seg.  Entering a sample with factor c_new multiplies it by c_cur / c_new
// (<= 1, so it never overflows); the final tile is multiplied by the last c.
#include "common.h"
#include "internal.h"

namespace dprc {

constexpr int kGM = 256, kGN = 256, kGK = 32;
// LDS: each operand column (an M or N index) holds its 32 tokens (64 B) in a
// row of 80 B; every 8 rows get 64 B more, so that the eight lanes of one LDS
// cycle hit distinct banks for both the transposing writes and the MFMA reads.
constexpr int kLdsRow = 80;
__host__ __device__ constexpr int lds_row_off(int r) { return r * kLdsRow + (r >> 3) * 64; }
constexpr int kLdsSide = lds_row_off(kGM);       // one operand tile (256 rows)
constexpr int kLdsStage = 2 * kLdsSide;          // both operands
constexpr int kLdsBytes = 2 * kLdsStage;         // two stages

__device__ __forceinline__ f32x4 mfma16g(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 tcol(const u32x4 (&rows)[8], int c) {
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

// MODE 0: clipped aggregation with split-K over the sorted active samples.
// MODE 1: FGC, z = sample, whole sample, no scaling.
template <int MODE>
__global__ void __launch_bounds__(256, 1) k_gemm_tokens(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ G, int T, int d, int p,
    const float* __restrict__ cvec, const int* __restrict__ order, const int* __restrict__ count,
    int64_t split_tokens, float* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int o0 = blockIdx.x * kGM;
  const int q0 = blockIdx.y * kGN;
  const int z = blockIdx.z;

  // Token range of this workgroup, as positions kv in the visiting order.
  int64_t kv0, kv1;
  if (MODE == 0) {
    const int64_t Kv = static_cast<int64_t>(*count) * T;
    kv0 = static_cast<int64_t>(z) * split_tokens;
    kv1 = kv0 + split_tokens < Kv ? kv0 + split_tokens : Kv;
  } else {
    kv0 = 0;
    kv1 = T;
  }
  float* dst = out + static_cast<int64_t>(z) * p * d;

  // Global loads: waves 0-1 fetch the G tile, waves 2-3 the A tile; each thread
  // one 8 x 8 unit (tokens 8 tg .. +7, columns 8 cg .. +7) per stage.
  const int side = tid >> 7;
  const int u = tid & 127;
  const int tg = u & 3, cg = u >> 2;
  const bf16_t* src = side == 0 ? G : A;
  const int ld = side == 0 ? p : d;
  const int c0 = side == 0 ? o0 : q0;
  uint32_t off[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) off[e] = static_cast<uint32_t>(((tg * 8 + e) * ld + cg * 8) * 2);
  unsigned char* lds_w = lds + side * kLdsSide + lds_row_off(cg * 8) + tg * 16;

  u32x4 rows[8];
  // Segment bookkeeping: stage kv lies in segment `seg` (a whole sample) at
  // token offset `seg_off`; T is a multiple of the stage size.
  int64_t ld_seg = kv0 / T;
  int ld_off = static_cast<int>(kv0 - ld_seg * T);
  auto gload = [&]() {
    const int64_t sample = MODE == 0 ? static_cast<int64_t>(order[ld_seg]) : static_cast<int64_t>(z);
    const unsigned char* base =
        reinterpret_cast<const unsigned char*>(src + (sample * T + ld_off) * ld + c0);
#pragma unroll
    for (int e = 0; e < 8; ++e) rows[e] = *reinterpret_cast<const u32x4*>(base + off[e]);
    ld_off += kGK;
    if (ld_off == T) {
      ld_off = 0;
      ++ld_seg;
    }
  };
  auto lstore = [&](int stage) {
    unsigned char* w = lds_w + stage * kLdsStage;
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4*>(w + c * kLdsRow) = tcol(rows, c);
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operand reads: lane (m, g) takes row m of each 16-row block, tokens 8 g .. +7.
  const int rd_lane = lds_row_off(m) + g * 16;
  auto compute = [&](int stage) {
    const unsigned char* sg = lds + stage * kLdsStage + lds_row_off(wm * 128) + rd_lane;
    const unsigned char* sa = lds + stage * kLdsStage + kLdsSide + lds_row_off(wn * 128) + rd_lane;
    u32x4 av[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) av[i] = *reinterpret_cast<const u32x4*>(sg + lds_row_off(16 * i));
    u32x4 bcur = *reinterpret_cast<const u32x4*>(sa);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 bnext = bcur;
      if (j < 7) bnext = *reinterpret_cast<const u32x4*>(sa + lds_row_off(16 * (j + 1)));
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i][j] = mfma16g(av[i], bcur, acc[i][j]);
      bcur = bnext;
    }
  };

  float cur_c = 1.f;
  int64_t cur_seg = -1;
  int64_t seg = kv0 / T;
  int seg_off = static_cast<int>(kv0 - seg * T);
  if (kv0 < kv1) {
    gload();
    lstore(0);
    __syncthreads();
    int stage = 0;
    for (int64_t kv = kv0; kv < kv1; kv += kGK) {
      const bool more = kv + kGK < kv1;
      if (more) gload();
      if (MODE == 0 && seg != cur_seg) {
        const float c_new = cvec[order[seg]];
        if (cur_seg >= 0) {
          const float ratio = cur_c / c_new;
          // In-place rescale, one 4-register block at a time; the empty asm
          // pins every block back to accumulator registers right away.
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              acc[i][j] *= ratio;
              asm volatile("" : "+a"(acc[i][j]));
            }
        }
        cur_c = c_new;
        cur_seg = seg;
      }
      compute(stage);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
      if (more) lstore(stage ^ 1);
      __syncthreads();
      stage ^= 1;
      seg_off += kGK;
      if (seg_off == T) {
        seg_off = 0;
        ++seg;
      }
    }
  }
  const float fin = (MODE == 0 && cur_seg >= 0) ? cur_c : 1.f;

  float* tile = dst + static_cast<int64_t>(o0 + wm * 128) * d + q0 + wn * 128;
  const uint32_t lane_off = static_cast<uint32_t>((4 * g * d + m) * 4);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      unsigned char* rowp = reinterpret_cast<unsigned char*>(tile + static_cast<int64_t>(i * 16 + r) * d);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float*>(rowp + lane_off + j * 64) = acc[i][j][r] * fin;
    }
}

bool mfma_gemm_ok(int T, int d, int p) {
  return T > 0 && T % kGK == 0 && d % kGN == 0 && p % kGM == 0;
}

// Split the token range so that there are about 256 workgroups.
int mfma_gemm_splits(int B, int T, int d, int p) {
  const int64_t tiles = static_cast<int64_t>(p / kGM) * (d / kGN);
  int64_t want = (256 + tiles - 1) / (tiles > 0 ? tiles : 1);
  const int64_t steps = static_cast<int64_t>(B) * T / kGK;
  if (want > steps) want = steps;
  if (want < 1) want = 1;
  return static_cast<int>(want);
}

// The 88 KiB LDS budget needs an explicit opt-in above the default limit.
template <int MODE>
static hipError_t set_lds_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_tokens<MODE>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
}

hipError_t launch_aggregate_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p,
                                 const float* c, const int* order, const int* count, int nsplit,
                                 float* part, hipStream_t s) {
  if (!mfma_gemm_ok(T, d, p) || nsplit < 1) return hipErrorInvalidValue;
  hipError_t e = set_lds_attr<0>();
  if (e != hipSuccess) return e;
  const int64_t total = static_cast<int64_t>(B) * T;
  int64_t per = (total + nsplit - 1) / nsplit;
  per = (per + kGK - 1) / kGK * kGK;
  hipLaunchKernelGGL(k_gemm_tokens<0>, dim3(p / kGM, d / kGN, nsplit), dim3(256), kLdsBytes, s, A,
                     G, T, d, p, c, order, count, per, part);
  return hipGetLastError();
}

hipError_t launch_fgc_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p, float* M,
                           hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!mfma_gemm_ok(T, d, p)) return hipErrorInvalidValue;
  hipError_t e = set_lds_attr<1>();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gemm_tokens<1>, dim3(p / kGM, d / kGN, B), dim3(256), kLdsBytes, s, A, G, T,
                     d, p, nullptr, nullptr, nullptr, static_cast<int64_t>(T), M);
  return hipGetLastError();
}

}  // namespace dprc
