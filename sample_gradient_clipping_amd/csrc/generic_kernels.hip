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
// sketch X = O S (classical Gram-Schmidt applied twice; any stable QR spans
// the same subspace, and the estimate depends only on that span), then the
// deflated tail probes W' = W - Q (Q^T W).  One block per sample.  Each thread
// owns the elements e = tid (mod blockDim) of every vector, so no thread ever
// reads global data another thread wrote; dot products reduce through LDS.
// ---------------------------------------------------------------------------
constexpr int kOrthMaxCols = 32;

__device__ void block_dots(double* h, int nd, double* red /*[16][kOrthMaxCols]*/) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int i = 0; i < nd; ++i) {
    const double v = wave_sum_d(h[i]);
    if (lane == 0) red[wid * kOrthMaxCols + i] = v;
  }
  __syncthreads();
  for (int i = 0; i < nd; ++i) {
    double t = 0.0;
    for (int w = 0; w < nw; ++w) t += red[w * kOrthMaxCols + i];
    h[i] = t;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(256) k_hpp_orth(const float* __restrict__ X, int xrows,
                                                  const float* __restrict__ Pw,
                                                  int64_t pw_bstride, int wrows, int p, int s_cols,
                                                  int r_cols, float* __restrict__ out) {
  __shared__ double red[16 * kOrthMaxCols];
  const int b = blockIdx.x;
  const float* xb = X + static_cast<int64_t>(b) * xrows * p;
  const float* wb = Pw + b * pw_bstride;
  float* ob = out + static_cast<int64_t>(b) * (s_cols + r_cols) * p;
  double h[kOrthMaxCols];
  for (int j = 0; j < s_cols; ++j) {
    float* qj = ob + static_cast<int64_t>(j) * p;
    for (int e = threadIdx.x; e < p; e += blockDim.x) qj[e] = xb[static_cast<int64_t>(j) * p + e];
    for (int pass = 0; pass < 2 && j > 0; ++pass) {
      for (int i = 0; i < j; ++i) h[i] = 0.0;
      for (int e = threadIdx.x; e < p; e += blockDim.x) {
        const double v = qj[e];
        for (int i = 0; i < j; ++i) h[i] += static_cast<double>(ob[static_cast<int64_t>(i) * p + e]) * v;
      }
      block_dots(h, j, red);
      for (int e = threadIdx.x; e < p; e += blockDim.x) {
        double v = qj[e];
        for (int i = 0; i < j; ++i) v -= h[i] * static_cast<double>(ob[static_cast<int64_t>(i) * p + e]);
        qj[e] = static_cast<float>(v);
      }
    }
    h[0] = 0.0;
    for (int e = threadIdx.x; e < p; e += blockDim.x) h[0] += static_cast<double>(qj[e]) * qj[e];
    block_dots(h, 1, red);
    const double nrm = sqrt(h[0]);
    const float inv = nrm > 0.0 ? static_cast<float>(1.0 / nrm) : 0.f;
    for (int e = threadIdx.x; e < p; e += blockDim.x) qj[e] *= inv;
  }
  for (int t = 0; t < r_cols; ++t) {
    const float* w = wb + static_cast<int64_t>(s_cols + t) * p;
    float* wo = ob + static_cast<int64_t>(s_cols + t) * p;
    for (int i = 0; i < s_cols; ++i) h[i] = 0.0;
    for (int e = threadIdx.x; e < p; e += blockDim.x) {
      const double v = w[e];
      for (int i = 0; i < s_cols; ++i) h[i] += static_cast<double>(ob[static_cast<int64_t>(i) * p + e]) * v;
    }
    block_dots(h, s_cols, red);
    for (int e = threadIdx.x; e < p; e += blockDim.x) {
      double v = w[e];
      for (int i = 0; i < s_cols; ++i) v -= h[i] * static_cast<double>(ob[static_cast<int64_t>(i) * p + e]);
      wo[e] = static_cast<float>(v);
    }
  }
  (void)wrows;
}

hipError_t launch_hpp_orth(const float* X, int xrows, const float* Pw, int64_t pw_bstride,
                           int wrows, int B, int p, int s_cols, int r_cols, float* out,
                           hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (s_cols > kOrthMaxCols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_hpp_orth, dim3(B), dim3(256), 0, s, X, xrows, Pw, pw_bstride, wrows, p,
                     s_cols, r_cols, out);
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
