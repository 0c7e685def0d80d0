// Per-sample gradients of the parameters that are not linear layers, on gfx950.
//
// RMSNorm gain (y_t = gamma * xhat_t): sample i's gradient in gamma is
// v_i = sum_t xhat_{i,t} * delta_{i,t} (delta = dl_i / dy), a column sum over
// the tokens; its squared norm joins n_i like any layer's (glossary page,
// section DP-SGDのアルゴリズム, steps 2-3: the whole per-sample gradient is
// clipped).  One streaming pass reads xhat and delta once (HBM-bound): a block
// owns 2048 columns (8 per thread, 16-byte loads for bf16) and a token split;
// the partial column sums of the splits are added in split order per sample,
// which also forms ||v_i||^2 in fp64.
#include "common.h"
#include "internal.h"

namespace dprc {

constexpr int kRmsThreads = 256;
constexpr int kRmsCols = 8;                           // columns per thread
constexpr int kRmsChunk = kRmsThreads * kRmsCols;     // columns per block
constexpr int kRmsUnroll = 8;                         // tokens in flight per thread

// 8 values of a row at column c0 (c0 + 8 <= d) as fp32.
__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(u[k] << 16);
    v[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// part[b][split][c] = sum over the split's tokens of xhat[b][t][c] * delta[b][t][c].
// VEC: d % 8 == 0 (vector loads); otherwise element loads with the column clamped.
template <typename TIn, bool VEC>
__global__ void __launch_bounds__(kRmsThreads) k_rmsnorm_partial(
    const TIn* __restrict__ X, const TIn* __restrict__ D, int T, int d, int tsplit,
    float* __restrict__ part) {
  const int b = blockIdx.z, split = blockIdx.y, nsplit = gridDim.y;
  const int c0 = blockIdx.x * kRmsChunk + threadIdx.x * kRmsCols;
  const int t0 = split * tsplit;
  const int t1 = t0 + tsplit < T ? t0 + tsplit : T;
  float acc[kRmsCols];
#pragma unroll
  for (int k = 0; k < kRmsCols; ++k) acc[k] = 0.f;
  const int cc = c0 < d ? c0 : 0;  // a thread past the last column reads column 0 and discards it
  const TIn* xb = X + (static_cast<int64_t>(b) * T) * d;
  const TIn* db = D + (static_cast<int64_t>(b) * T) * d;
  auto row = [&](int t, float (&xv)[8], float (&dv)[8]) {
    if (VEC) {
      load8(xb + static_cast<int64_t>(t) * d + cc, xv);
      load8(db + static_cast<int64_t>(t) * d + cc, dv);
    } else {
#pragma unroll
      for (int k = 0; k < kRmsCols; ++k) {
        const int c = cc + k < d ? cc + k : d - 1;
        xv[k] = load_f32(xb + static_cast<int64_t>(t) * d + c);
        dv[k] = load_f32(db + static_cast<int64_t>(t) * d + c);
      }
    }
  };
  int t = t0;
  for (; t + kRmsUnroll <= t1; t += kRmsUnroll) {
    float xv[kRmsUnroll][8], dv[kRmsUnroll][8];
#pragma unroll
    for (int u = 0; u < kRmsUnroll; ++u) row(t + u, xv[u], dv[u]);
#pragma unroll
    for (int u = 0; u < kRmsUnroll; ++u)
#pragma unroll
      for (int k = 0; k < kRmsCols; ++k) acc[k] = fmaf(xv[u][k], dv[u][k], acc[k]);
  }
  for (; t < t1; ++t) {
    float xv[8], dv[8];
    row(t, xv, dv);
#pragma unroll
    for (int k = 0; k < kRmsCols; ++k) acc[k] = fmaf(xv[k], dv[k], acc[k]);
  }
  if (c0 >= d) return;
  float* pb = part + (static_cast<int64_t>(b) * nsplit + split) * d + c0;
#pragma unroll
  for (int k = 0; k < kRmsCols; ++k)
    if (c0 + k < d) pb[k] = acc[k];
}

// v[b][c] = sum_split part[b][split][c] (split order, eight loads in flight,
// split index clamped: no load under a condition); sq[b][chunk] = sum over the
// block's 256 columns of v^2 (fp64).
constexpr int kRmsRed = 256;
__global__ void __launch_bounds__(kRmsRed) k_rmsnorm_reduce(const float* __restrict__ part,
                                                           int nsplit, int d,
                                                           float* __restrict__ v,
                                                           double* __restrict__ sq) {
  __shared__ double red[16];
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int c = chunk * kRmsRed + threadIdx.x;
  const int cc = c < d ? c : d - 1;
  const float* pb = part + static_cast<int64_t>(b) * nsplit * d + cc;
  float s = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = s0 + u < nsplit ? s0 + u : nsplit - 1;
      x[u] = pb[static_cast<int64_t>(sp) * d];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s += s0 + u < nsplit ? x[u] : 0.f;
  }
  if (c < d && v) v[static_cast<int64_t>(b) * d + c] = s;
  const double q = c < d ? static_cast<double>(s) * s : 0.0;
  const double t = block_sum_d(q, red);
  if (threadIdx.x == 0) sq[static_cast<int64_t>(b) * gridDim.x + chunk] = t;
}

// n_sq[b] (= or +=) sum_chunk sq[b][chunk] in chunk order.
__global__ void k_rmsnorm_final(const double* __restrict__ sq, int nchunk, float* __restrict__ n_sq,
                                int accumulate, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  double t = 0.0;
  for (int k = 0; k < nchunk; ++k) t += sq[static_cast<int64_t>(b) * nchunk + k];
  n_sq[b] = static_cast<float>(accumulate ? static_cast<double>(n_sq[b]) + t : t);
}

int rmsnorm_splits(int B, int T, int d) {
  const int chunks = (d + kRmsChunk - 1) / kRmsChunk;
  int want = (512 + B * chunks - 1) / (B * chunks > 0 ? B * chunks : 1);
  const int maxs = T / 32 > 0 ? T / 32 : 1;  // at least 32 tokens per split
  if (want > maxs) want = maxs;
  return want < 1 ? 1 : want;
}

__global__ void k_rmsnorm_empty(int d, float* __restrict__ v, double* __restrict__ sq) {
  const int b = blockIdx.y, c = blockIdx.x * kRmsRed + threadIdx.x;
  if (v && c < d) v[static_cast<int64_t>(b) * d + c] = 0.f;
  if (threadIdx.x == 0) sq[static_cast<int64_t>(b) * gridDim.x + blockIdx.x] = 0.0;
}

int rmsnorm_sq_chunks(int d) { return (d + kRmsRed - 1) / kRmsRed; }

template <typename TIn>
hipError_t launch_rmsnorm_norm(const TIn* X, const TIn* D, int B, int T, int d, float* part,
                               int nsplit, double* sq, float* v, float* n_sq, int accumulate,
                               hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (T > 0) {
    const int tsplit = (T + nsplit - 1) / nsplit;
    const dim3 grid((d + kRmsChunk - 1) / kRmsChunk, nsplit, B);
    const bool vec = d % 8 == 0;
    if (vec)
      hipLaunchKernelGGL((k_rmsnorm_partial<TIn, true>), grid, dim3(kRmsThreads), 0, s, X, D, T, d,
                         tsplit, part);
    else
      hipLaunchKernelGGL((k_rmsnorm_partial<TIn, false>), grid, dim3(kRmsThreads), 0, s, X, D, T,
                         d, tsplit, part);
  } else {
    nsplit = 0;  // no tokens: v = 0, n += 0
  }
  const int nchunk = (d + kRmsRed - 1) / kRmsRed;
  if (nsplit > 0) {
    hipLaunchKernelGGL(k_rmsnorm_reduce, dim3(nchunk, B), dim3(kRmsRed), 0, s, part, nsplit, d,
                       v, sq);
  } else {
    // no tokens: v = 0 and every chunk contributes 0
    hipLaunchKernelGGL(k_rmsnorm_empty, dim3(nchunk, B), dim3(kRmsRed), 0, s, d, v, sq);
  }
  hipLaunchKernelGGL(k_rmsnorm_final, dim3((B + 63) / 64), dim3(64), 0, s, sq, nchunk, n_sq,
                     accumulate, B);
  return hipGetLastError();
}

// S[c] = sum_i c_i v[i][c] (sample order).
__global__ void k_weighted_rows(const float* __restrict__ v, const float* __restrict__ c, int B,
                                int d, float* __restrict__ S) {
  const int col = blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= d) return;
  float s = 0.f;
  for (int i = 0; i < B; ++i) s = fmaf(c[i], v[static_cast<int64_t>(i) * d + col], s);
  S[col] = s;
}

hipError_t launch_weighted_rows(const float* v, const float* c, int B, int d, float* S,
                                hipStream_t s) {
  if (d <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_weighted_rows, dim3((d + 255) / 256), dim3(256), 0, s, v, c, B, d, S);
  return hipGetLastError();
}

template hipError_t launch_rmsnorm_norm<float>(const float*, const float*, int, int, int, float*,
                                               int, double*, float*, float*, int, hipStream_t);
template hipError_t launch_rmsnorm_norm<bf16_t>(const bf16_t*, const bf16_t*, int, int, int,
                                                float*, int, double*, float*, float*, int,
                                                hipStream_t);

}  // namespace dprc
