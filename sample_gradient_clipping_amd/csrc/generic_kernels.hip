// Generic HIP kernels for gfx950: any shape, fp32 or bf16 inputs, fp32 math.
// They serve fp32 inputs and bf16 shapes outside the MFMA tilings, and hold
// the small glue steps (clip, reductions, Hutch++ orthonormalisation) that
// both paths share.  One thread per output and a plain loop over the
// contracted index: simple, deterministic, and exact up to fp32 rounding.
#include "common.h"
#include "internal.h"

namespace dprc {

static inline unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

// ---------------------------------------------------------------------------
// Hutchinson thin products (the randomized-clipping summary, section
// 中核メカニズム, item 1): Y = G P along the row, Z = A^T Y along the tokens.
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ void k_sketch_generic(const TIn* __restrict__ X, int T, int W,
                                 const float* __restrict__ P, int64_t p_bstride, int kp,
                                 float* __restrict__ Y) {
  const int b = blockIdx.y;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(kp) * T) return;
  const int j = static_cast<int>(idx / T), t = static_cast<int>(idx % T);
  const TIn* x = X + (static_cast<int64_t>(b) * T + t) * W;
  const float* pr = P + b * p_bstride + static_cast<int64_t>(j) * W;
  float acc = 0.f;
  for (int r = 0; r < W; ++r) acc = fmaf(load_f32(x + r), pr[r], acc);
  Y[(static_cast<int64_t>(b) * kp + j) * T + t] = acc;
}

template <typename TIn>
hipError_t launch_sketch_generic(const TIn* X, int B, int T, int W, const float* P,
                                 int64_t p_bstride, int kp, float* Y, hipStream_t s) {
  if (B <= 0 || T <= 0 || kp <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sketch_generic<TIn>, dim3(cdiv(static_cast<int64_t>(kp) * T, 256), B),
                     dim3(256), 0, s, X, T, W, P, p_bstride, kp, Y);
  return hipGetLastError();
}

template <typename TIn>
__global__ void k_project_generic(const TIn* __restrict__ X, int T, int W,
                                  const float* __restrict__ Y, int kp, float* __restrict__ Z) {
  const int b = blockIdx.y;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(kp) * W) return;
  const int j = static_cast<int>(idx / W), q = static_cast<int>(idx % W);
  const TIn* x = X + static_cast<int64_t>(b) * T * W + q;
  const float* y = Y + (static_cast<int64_t>(b) * kp + j) * T;
  float acc = 0.f;
  for (int t = 0; t < T; ++t) acc = fmaf(load_f32(x + static_cast<int64_t>(t) * W), y[t], acc);
  Z[(static_cast<int64_t>(b) * kp + j) * W + q] = acc;
}

template <typename TIn>
hipError_t launch_project_generic(const TIn* X, int B, int T, int W, const float* Y, int kp,
                                  float* Z, hipStream_t s) {
  if (B <= 0 || kp <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_project_generic<TIn>, dim3(cdiv(static_cast<int64_t>(kp) * W, 256), B),
                     dim3(256), 0, s, X, T, W, Y, kp, Z);
  return hipGetLastError();
}

// Weighted sum of squares of the split-summed Z, in fp64, one partial per block.
__global__ void __launch_bounds__(256) k_frob_partial(const float* __restrict__ Z, int nsplit,
                                                      int kp, int W, int n0, float w0, int n1,
                                                      float w1, double* __restrict__ part,
                                                      int nchunk) {
  __shared__ double red[16];
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int64_t E = static_cast<int64_t>(kp) * W;
  const int64_t per = (E + nchunk - 1) / nchunk;
  const int64_t e0 = chunk * per, e1 = (e0 + per < E) ? e0 + per : E;
  const float* zb = Z + static_cast<int64_t>(b) * nsplit * E;
  double acc = 0.0;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += blockDim.x) {
    const int j = static_cast<int>(e / W);
    const float w = j < n0 ? w0 : (j < n0 + n1 ? w1 : 0.f);
    if (w == 0.f) continue;
    float z = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) z += zb[sp * E + e];
    acc += static_cast<double>(w) * static_cast<double>(z) * static_cast<double>(z);
  }
  acc = block_sum_d(acc, red);
  if (threadIdx.x == 0) part[static_cast<int64_t>(b) * nchunk + chunk] = acc;
}

hipError_t launch_frob_partial(const float* Z, int B, int nsplit, int kp, int W, int n0, float w0,
                               int n1, float w1, double* part, int nchunk, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_frob_partial, dim3(nchunk, B), dim3(256), 0, s, Z, nsplit, kp, W, n0, w0,
                     n1, w1, part, nchunk);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) k_sum_parts(const double* __restrict__ part, int nparts,
                                                   float* __restrict__ n, int accumulate) {
  __shared__ double red[16];
  const int b = blockIdx.x;
  double acc = 0.0;
  for (int c = threadIdx.x; c < nparts; c += blockDim.x) acc += part[static_cast<int64_t>(b) * nparts + c];
  acc = block_sum_d(acc, red);
  if (threadIdx.x == 0) n[b] = static_cast<float>(accumulate ? static_cast<double>(n[b]) + acc : acc);
}

hipError_t launch_sum_parts(const double* part, int B, int nparts, float* n, int accumulate,
                            hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sum_parts, dim3(B), dim3(256), 0, s, part, nparts, n, accumulate);
  return hipGetLastError();
}

__global__ void k_sum_splits(const float* __restrict__ Zp, int nsplit, int rows, int W,
                             float* __restrict__ Z, bf16_t* __restrict__ Zb) {
  const int b = blockIdx.y;
  const int64_t E = static_cast<int64_t>(rows) * W;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E) return;
  float z = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) z += Zp[(static_cast<int64_t>(b) * nsplit + sp) * E + e];
  if (Z) Z[static_cast<int64_t>(b) * E + e] = z;
  if (Zb) Zb[static_cast<int64_t>(b) * E + e] = f32_to_bf16(z);
}

hipError_t launch_sum_splits(const float* Zp, int B, int nsplit, int rows, int W, float* Z,
                             bf16_t* Zb, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sum_splits, dim3(cdiv(static_cast<int64_t>(rows) * W, 256), B), dim3(256),
                     0, s, Zp, nsplit, rows, W, Z, Zb);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Ghost clipping baseline: sum over token pairs of (A A^T)_{st} (G G^T)_{st},
// upper triangle counted twice (summary, sections 問題定義 / 複雑性の削減).
// ---------------------------------------------------------------------------
int ghost_generic_nparts(int T) {
  return static_cast<int>(cdiv(static_cast<int64_t>(T) * T, 256));
}

template <typename TIn>
__global__ void __launch_bounds__(256) k_ghost_generic(const TIn* __restrict__ A,
                                                       const TIn* __restrict__ G, int T, int d,
                                                       int p, double* __restrict__ part) {
  __shared__ double red[16];
  const int b = blockIdx.y;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  double v = 0.0;
  if (idx < static_cast<int64_t>(T) * T) {
    const int s0 = static_cast<int>(idx / T), t0 = static_cast<int>(idx % T);
    if (s0 <= t0) {
      const TIn* as = A + (static_cast<int64_t>(b) * T + s0) * d;
      const TIn* at = A + (static_cast<int64_t>(b) * T + t0) * d;
      const TIn* gs = G + (static_cast<int64_t>(b) * T + s0) * p;
      const TIn* gt = G + (static_cast<int64_t>(b) * T + t0) * p;
      float ga = 0.f, gg = 0.f;
      for (int q = 0; q < d; ++q) ga = fmaf(load_f32(as + q), load_f32(at + q), ga);
      for (int o = 0; o < p; ++o) gg = fmaf(load_f32(gs + o), load_f32(gt + o), gg);
      v = static_cast<double>(ga) * static_cast<double>(gg) * (s0 == t0 ? 1.0 : 2.0);
    }
  }
  v = block_sum_d(v, red);
  if (threadIdx.x == 0) part[static_cast<int64_t>(b) * gridDim.x + blockIdx.x] = v;
}

template <typename TIn>
hipError_t launch_ghost_generic(const TIn* A, const TIn* G, int B, int T, int d, int p,
                                double* part, int* nparts_out, hipStream_t s) {
  const int np = ghost_generic_nparts(T);
  *nparts_out = np;
  if (B <= 0 || np == 0) return hipSuccess;
  hipLaunchKernelGGL(k_ghost_generic<TIn>, dim3(np, B), dim3(256), 0, s, A, G, T, d, p, part);
  return hipGetLastError();
}

// FGC baseline: materialise M_b[o][q] = sum_t G_b[t][o] A_b[t][q].
template <typename TIn>
__global__ void k_fgc_generic(const TIn* __restrict__ A, const TIn* __restrict__ G, int T, int d,
                              int p, float* __restrict__ M) {
  const int b = blockIdx.y;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(p) * d) return;
  const int o = static_cast<int>(idx / d), q = static_cast<int>(idx % d);
  const TIn* a = A + static_cast<int64_t>(b) * T * d + q;
  const TIn* g = G + static_cast<int64_t>(b) * T * p + o;
  float acc = 0.f;
  for (int t = 0; t < T; ++t)
    acc = fmaf(load_f32(g + static_cast<int64_t>(t) * p), load_f32(a + static_cast<int64_t>(t) * d), acc);
  M[static_cast<int64_t>(b) * p * d + idx] = acc;
}

template <typename TIn>
hipError_t launch_fgc_generic(const TIn* A, const TIn* G, int B, int T, int d, int p, float* M,
                              hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fgc_generic<TIn>, dim3(cdiv(static_cast<int64_t>(p) * d, 256), B),
                     dim3(256), 0, s, A, G, T, d, p, M);
  return hipGetLastError();
}

// Clipped sum S[o][q] = sum_b c_b sum_t G_b[t][o] A_b[t][q]; each sample is
// summed in fp32 and scaled once (dropped samples, c_b = 0, are skipped).
template <typename TIn>
__global__ void k_aggregate_generic(const TIn* __restrict__ A, const TIn* __restrict__ G, int B,
                                    int T, int d, int p, const float* __restrict__ c,
                                    float* __restrict__ S) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(p) * d) return;
  const int o = static_cast<int>(idx / d), q = static_cast<int>(idx % d);
  float total = 0.f;
  for (int b = 0; b < B; ++b) {
    const float cb = c[b];
    if (cb == 0.f) continue;
    const TIn* a = A + static_cast<int64_t>(b) * T * d + q;
    const TIn* g = G + static_cast<int64_t>(b) * T * p + o;
    float acc = 0.f;
    for (int t = 0; t < T; ++t)
      acc = fmaf(load_f32(g + static_cast<int64_t>(t) * p), load_f32(a + static_cast<int64_t>(t) * d), acc);
    total = fmaf(cb, acc, total);
  }
  S[idx] = total;
}

template <typename TIn>
hipError_t launch_aggregate_generic(const TIn* A, const TIn* G, int B, int T, int d, int p,
                                    const float* c, float* S, hipStream_t s) {
  hipLaunchKernelGGL(k_aggregate_generic<TIn>, dim3(cdiv(static_cast<int64_t>(p) * d, 256)),
                     dim3(256), 0, s, A, G, B, T, d, p, c, S);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Clip factors (glossary page, section DP-SGDのアルゴリズム, step 3; summary,
// section アルゴリズム的フロー, step 4): c = 1 if n <= C^2, C / sqrt(n) above,
// 0 for a non-finite n (flagged).  Also lists the active samples (c > 0) in
// ascending (c, index) order for the MFMA aggregation.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float clip_of(float v, float C) {
  if (!isfinite(v)) return 0.f;
  if (v <= C * C) return 1.f;
  return C / sqrtf(v);
}

__global__ void __launch_bounds__(1024) k_clip(const float* __restrict__ n, int B, float C,
                                               float* __restrict__ c, float* __restrict__ c_out,
                                               uint32_t* __restrict__ status,
                                               int* __restrict__ order, int* __restrict__ count) {
  __shared__ int s_count;
  __shared__ int s_bad;
  if (threadIdx.x == 0) {
    s_count = 0;
    s_bad = 0;
  }
  __syncthreads();
  int local = 0, bad = 0;
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const float v = n[i];
    const float ci = clip_of(v, C);
    c[i] = ci;
    if (c_out) c_out[i] = ci;
    if (!isfinite(v)) bad = 1;
    if (ci > 0.f) {
      ++local;
      int rank = 0;
      for (int j = 0; j < B; ++j) {
        const float cj = clip_of(n[j], C);
        rank += (cj > 0.f) && (cj < ci || (cj == ci && j < i));
      }
      order[rank] = i;
    }
  }
  atomicAdd(&s_count, local);
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    *count = s_count;
    if (s_bad && status) atomicOr(status, DPRC_STATUS_NONFINITE);
  }
}

hipError_t launch_clip(const float* n, int B, float C, float* c, float* c_out, uint32_t* status,
                       int* order, int* count, hipStream_t s) {
  hipLaunchKernelGGL(k_clip, dim3(1), dim3(1024), 0, s, n, B, C, c, c_out, status, order, count);
  return hipGetLastError();
}

// out[e] = sum over splits of part[split][e], fixed order.
__global__ void k_reduce_splits(const float* __restrict__ part, int nsplit, int64_t n,
                                float* __restrict__ out) {
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (e0 >= n) return;
  if (e0 + 3 < n) {
    float4 acc = *reinterpret_cast<const float4*>(part + e0);
    for (int sp = 1; sp < nsplit; ++sp) {
      const float4 v = *reinterpret_cast<const float4*>(part + sp * n + e0);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *reinterpret_cast<float4*>(out + e0) = acc;
  } else {
    for (int64_t e = e0; e < n; ++e) {
      float acc = 0.f;
      for (int sp = 0; sp < nsplit; ++sp) acc += part[sp * n + e];
      out[e] = acc;
    }
  }
}

hipError_t launch_reduce_splits(const float* part, int nsplit, int64_t n, float* out,
                                hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_reduce_splits, dim3(cdiv((n + 3) / 4, 256)), dim3(256), 0, s, part, nsplit,
                     n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Hutch++ (summary, section 中核メカニズム, item 2): orthonormal basis Q of the
// sketch X = O S, then the deflated tail probes W' = W - Q (Q^T W).  Any
// stable QR spans the same subspace and the estimate depends only on that
// span; this one is CholeskyQR2 (Gram matrix and Cholesky factor in fp64,
// applied twice).  A pivot that vanishes relative to the largest one (rank
// deficiency) zeroes its column of Q; the remaining columns still span
// range(X) and Q Q^T is the orthogonal projector onto it.  The vectors of
// length p are rows here (X^T's columns).  Work is split over chunks of
// kOrthChunk elements of p so that every step has many blocks:
//   k_orth_dots    partial inner products of row sets over one chunk;
//   k_orth_apply   sums the partials in a fixed order, factors the Gram
//                  (redundantly per block; tiny) and writes Q = rows R^-1;
//   k_orth_deflate W' = W - Q H from the summed partial products H = Q W^T.
// ---------------------------------------------------------------------------
constexpr int kOrthMaxCols = 32;
constexpr int kOrthChunk = 256;

int orth_chunks(int p) { return (p + kOrthChunk - 1) / kOrthChunk; }

// part[b][chunk][i * nv + j] = sum_{e in chunk} U[i][e] V[j][e], fp64.
__global__ void __launch_bounds__(kOrthChunk) k_orth_dots(
    const float* __restrict__ U, int64_t u_bstride, int nu, const float* __restrict__ V,
    int64_t v_bstride, int nv, int p, double* __restrict__ part) {
  __shared__ float su[kOrthMaxCols][kOrthChunk];
  __shared__ float sv[kOrthMaxCols][kOrthChunk];
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int e0 = chunk * kOrthChunk;
  const int e = e0 + threadIdx.x;
  const float* ub = U + b * u_bstride;
  const float* vb = V + b * v_bstride;
  // all loads first, then the LDS stores (one memory round trip, not one per row)
  float ru[kOrthMaxCols], rv[kOrthMaxCols];
#pragma unroll
  for (int i = 0; i < kOrthMaxCols; ++i) {
    ru[i] = (i < nu && e < p) ? ub[static_cast<int64_t>(i) * p + e] : 0.f;
    rv[i] = (i < nv && e < p) ? vb[static_cast<int64_t>(i) * p + e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kOrthMaxCols; ++i) {
    if (i < nu) su[i][threadIdx.x] = ru[i];
    if (i < nv) sv[i][threadIdx.x] = rv[i];
  }
  __syncthreads();
  const int npairs = nu * nv;
  double* out = part + (static_cast<int64_t>(b) * gridDim.x + chunk) * npairs;
  for (int pi = threadIdx.x; pi < npairs; pi += blockDim.x) {
    const int i = pi / nv, j = pi % nv;
    double acc = 0.0;
    for (int t = 0; t < kOrthChunk; ++t)
      acc += static_cast<double>(su[i][t]) * static_cast<double>(sv[j][t]);
    out[pi] = acc;
  }
}

// Sum of the chunk partials of one sample into LDS dst[npairs], each entry
// added up in chunk order.  The partials are contiguous ([chunk][pair]), so
// tiles of whole chunks are first copied into LDS with every thread loading
// (one memory round trip per tile), then summed from LDS.
constexpr int kSumStage = 4096;  // doubles of LDS staging
__device__ void sum_chunks(const double* part_b, int nchunk, int npairs, double* dst,
                           double* stage) {
  for (int pi = threadIdx.x; pi < npairs; pi += blockDim.x) dst[pi] = 0.0;
  const int tile = npairs < kSumStage ? kSumStage / npairs : 1;
  for (int c0 = 0; c0 < nchunk; c0 += tile) {
    const int nc = nchunk - c0 < tile ? nchunk - c0 : tile;
    __syncthreads();
    // sixteen loads in flight per thread before the first LDS store
    const int n = nc * npairs;
    const double* src = part_b + static_cast<int64_t>(c0) * npairs;
    for (int u0 = 0; u0 < n; u0 += 16 * blockDim.x) {
      double v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int u = u0 + k * blockDim.x + threadIdx.x;
        v[k] = u < n ? src[u] : 0.0;
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int u = u0 + k * blockDim.x + threadIdx.x;
        if (u < n) stage[u] = v[k];
      }
    }
    __syncthreads();
    for (int pi = threadIdx.x; pi < npairs; pi += blockDim.x) {
      double acc = dst[pi];
      for (int c = 0; c < nc; ++c) acc += stage[c * npairs + pi];
      dst[pi] = acc;
    }
  }
}

// Cholesky of the s x s Gram (dense, gram[i * s + j]; overwritten) and the
// inverse of its factor, fp64, by the whole block (LDS arrays, one
// synchronisation per step).  Right-looking: at step j the pivot row is
// scaled and the trailing upper triangle is updated, so every entry receives
// its rank-one corrections in the same order as the textbook left-looking
// form.  A pivot that is not above tiny = 1e-24 * (largest diagonal) marks
// column j dead: its row and column of R and of R^-1 are zero.
__device__ void chol_inverse(double* gram, int s, double (*R)[kOrthMaxCols],
                             double (*Rinv)[kOrthMaxCols], double* tiny_s, uint32_t* dead_s) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (tid == 0) {
    double dmax = 0.0;
    for (int i = 0; i < s; ++i) dmax = fmax(dmax, gram[i * s + i]);
    *tiny_s = dmax * 1e-24;
    *dead_s = 0u;
  }
  for (int u = tid; u < kOrthMaxCols * kOrthMaxCols; u += nt) {
    R[u / kOrthMaxCols][u % kOrthMaxCols] = 0.0;
    Rinv[u / kOrthMaxCols][u % kOrthMaxCols] = 0.0;
  }
  __syncthreads();
  for (int j = 0; j < s; ++j) {
    const double djj = gram[j * s + j];
    const bool dj = !(djj > *tiny_s);
    const double rjj = dj ? 0.0 : sqrt(djj);
    const double inv = dj ? 0.0 : 1.0 / rjj;
    // row j of R
    for (int c = j + tid; c < s; c += nt) R[j][c] = c == j ? rjj : gram[j * s + c] * inv;
    if (tid == 0 && dj) *dead_s |= 1u << j;
    __syncthreads();
    // trailing update of the upper triangle: gram[i][c] -= R[j][i] R[j][c], j < i <= c
    const int m = s - j - 1;
    for (int u = tid; u < m * m; u += nt) {
      const int i = j + 1 + u / m, c = j + 1 + u % m;
      if (c >= i) gram[i * s + c] -= R[j][i] * R[j][c];
    }
    __syncthreads();
  }
  // R^-1 (upper triangular): lane j back-substitutes column j.
  const uint32_t dead = *dead_s;
  for (int j = tid; j < s; j += nt) {
    if (dead >> j & 1u) continue;
    for (int i = j; i >= 0; --i) {
      if (dead >> i & 1u) continue;
      double v = i == j ? 1.0 : 0.0;
      for (int k = i + 1; k <= j; ++k) v -= R[i][k] * Rinv[k][j];
      Rinv[i][j] = v / R[i][i];
    }
  }
  __syncthreads();
}

// Q[j][e] = sum_{i <= j} X[i][e] Rinv[i][j], Rinv from the Gram partials of X.
__global__ void __launch_bounds__(kOrthChunk) k_orth_apply(
    const float* __restrict__ Xr, int64_t x_bstride, int s, int p,
    const double* __restrict__ part, int nchunk, float* __restrict__ Q, int64_t q_bstride) {
  __shared__ double gram[kOrthMaxCols * kOrthMaxCols];
  __shared__ double R[kOrthMaxCols][kOrthMaxCols];
  __shared__ double Rinv[kOrthMaxCols][kOrthMaxCols];
  __shared__ double stage[kSumStage];
  __shared__ double tiny;
  __shared__ uint32_t dead;
  const int b = blockIdx.y;
  sum_chunks(part + static_cast<int64_t>(b) * nchunk * s * s, nchunk, s * s, gram, stage);
  __syncthreads();
  chol_inverse(gram, s, R, Rinv, &tiny, &dead);
  const int e = blockIdx.x * kOrthChunk + threadIdx.x;
  if (e >= p) return;
  const float* xb = Xr + b * x_bstride;
  float* qb = Q + b * q_bstride;
  float x[kOrthMaxCols];
#pragma unroll
  for (int i = 0; i < kOrthMaxCols; ++i) x[i] = i < s ? xb[static_cast<int64_t>(i) * p + e] : 0.f;
#pragma unroll
  for (int j = 0; j < kOrthMaxCols; ++j) {
    if (j < s) {
      double q = 0.0;
#pragma unroll
      for (int i = 0; i <= j; ++i) q += static_cast<double>(x[i]) * Rinv[i][j];
      qb[static_cast<int64_t>(j) * p + e] = static_cast<float>(q);
    }
  }
}

// W'[t][e] = W[t][e] - sum_i H[i][t] Q[i][e], H = summed partials of Q W^T.
__global__ void __launch_bounds__(kOrthChunk) k_orth_deflate(
    const float* __restrict__ Q, int64_t q_bstride, int s, const float* __restrict__ W,
    int64_t w_bstride, int r, int p, const double* __restrict__ part, int nchunk,
    float* __restrict__ Wout, int64_t wo_bstride) {
  __shared__ double H[kOrthMaxCols * kOrthMaxCols];
  __shared__ double stage[kSumStage];
  const int b = blockIdx.y;
  sum_chunks(part + static_cast<int64_t>(b) * nchunk * s * r, nchunk, s * r, H, stage);
  __syncthreads();
  const int e = blockIdx.x * kOrthChunk + threadIdx.x;
  if (e >= p) return;
  const float* qb = Q + b * q_bstride;
  const float* wb = W + b * w_bstride;
  float* ob = Wout + b * wo_bstride;
  float q[kOrthMaxCols], w[kOrthMaxCols];
#pragma unroll
  for (int i = 0; i < kOrthMaxCols; ++i) {
    q[i] = i < s ? qb[static_cast<int64_t>(i) * p + e] : 0.f;
    w[i] = i < r ? wb[static_cast<int64_t>(i) * p + e] : 0.f;
  }
#pragma unroll
  for (int t = 0; t < kOrthMaxCols; ++t) {
    if (t < r) {
      double v = w[t];
#pragma unroll
      for (int i = 0; i < kOrthMaxCols; ++i)
        if (i < s) v -= H[i * r + t] * static_cast<double>(q[i]);
      ob[static_cast<int64_t>(t) * p + e] = static_cast<float>(v);
    }
  }
}

size_t hpp_orth_scratch_bytes(int B, int p, int s, int r) {
  const int npairs = s * s > s * r ? s * s : s * r;
  return static_cast<size_t>(B) * orth_chunks(p) * (npairs > 0 ? npairs : 1) * sizeof(double);
}

hipError_t launch_hpp_orth(const float* X, int xrows, const float* Pw, int64_t pw_bstride,
                           int wrows, int B, int p, int s_cols, int r_cols, float* out,
                           double* scratch, hipStream_t st) {
  (void)wrows;
  if (B <= 0) return hipSuccess;
  if (s_cols < 1 || s_cols > kOrthMaxCols || r_cols > kOrthMaxCols) return hipErrorInvalidValue;
  const int nch = orth_chunks(p);
  const int64_t xs = static_cast<int64_t>(xrows) * p;
  const int64_t os = static_cast<int64_t>(s_cols + r_cols) * p;
  const dim3 grid(nch, B);
  // pass 1: Q1 = X R1^-1
  hipLaunchKernelGGL(k_orth_dots, grid, dim3(kOrthChunk), 0, st, X, xs, s_cols, X, xs, s_cols, p,
                     scratch);
  hipLaunchKernelGGL(k_orth_apply, grid, dim3(kOrthChunk), 0, st, X, xs, s_cols, p, scratch, nch,
                     out, os);
  // pass 2: Q = Q1 R2^-1 (in place: each thread reads its element before writing it)
  hipLaunchKernelGGL(k_orth_dots, grid, dim3(kOrthChunk), 0, st, out, os, s_cols, out, os, s_cols,
                     p, scratch);
  hipLaunchKernelGGL(k_orth_apply, grid, dim3(kOrthChunk), 0, st, out, os, s_cols, p, scratch, nch,
                     out, os);
  if (r_cols > 0) {
    const float* W = Pw + static_cast<int64_t>(s_cols) * p;  // tail probe rows s .. s+r-1
    hipLaunchKernelGGL(k_orth_dots, grid, dim3(kOrthChunk), 0, st, out, os, s_cols, W, pw_bstride,
                       r_cols, p, scratch);
    hipLaunchKernelGGL(k_orth_deflate, grid, dim3(kOrthChunk), 0, st, out, os, s_cols, W,
                       pw_bstride, r_cols, p, scratch, nch, out + static_cast<int64_t>(s_cols) * p,
                       os);
  }
  return hipGetLastError();
}

__global__ void k_to_bf16_pad(const float* __restrict__ in, int rows_in, int rows_out, int W,
                              bf16_t* __restrict__ out) {
  const int b = blockIdx.y;
  const int64_t E = static_cast<int64_t>(rows_out) * W;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int j = static_cast<int>(e / W);
  const float v = j < rows_in ? in[(static_cast<int64_t>(b) * rows_in) * W + e] : 0.f;
  out[static_cast<int64_t>(b) * E + e] = f32_to_bf16(v);
}

hipError_t launch_to_bf16_pad(const float* in, int B, int rows_in, int rows_out, int W,
                              bf16_t* out, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_to_bf16_pad, dim3(cdiv(static_cast<int64_t>(rows_out) * W, 256), B),
                     dim3(256), 0, s, in, rows_in, rows_out, W, out);
  return hipGetLastError();
}

#define DPRC_INSTANTIATE(TIn)                                                                      \
  template hipError_t launch_sketch_generic<TIn>(const TIn*, int, int, int, const float*, int64_t, \
                                                 int, float*, hipStream_t);                        \
  template hipError_t launch_project_generic<TIn>(const TIn*, int, int, int, const float*, int,    \
                                                  float*, hipStream_t);                            \
  template hipError_t launch_ghost_generic<TIn>(const TIn*, const TIn*, int, int, int, int,        \
                                                double*, int*, hipStream_t);                       \
  template hipError_t launch_fgc_generic<TIn>(const TIn*, const TIn*, int, int, int, int, float*,  \
                                              hipStream_t);                                        \
  template hipError_t launch_aggregate_generic<TIn>(const TIn*, const TIn*, int, int, int, int,    \
                                                    const float*, float*, hipStream_t);
DPRC_INSTANTIATE(float)
DPRC_INSTANTIATE(bf16_t)

}  // namespace dprc
