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

// Measurement hook: a plain streaming read of n16 16-byte words, the
// practical HBM read ceiling the bandwidth-bound kernels are compared with.
// Workgroup x reads words x * 256 * kReadUnroll + ... grid-stride, eight 16-byte
// loads per thread in flight, and writes the XOR of everything it read to
// out[x] (so that no load can be dropped, and the result can be checked).
constexpr int kReadUnroll = 8;

__global__ void __launch_bounds__(256) k_stream_read(const u32x4* __restrict__ in, int64_t n16,
                                                     uint32_t* __restrict__ out) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t step = static_cast<int64_t>(gridDim.x) * 256 * kReadUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * kReadUnroll + threadIdx.x; base < n16;
       base += step) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t i = base + u * 256;
      v[u] = in[i < n16 ? i : n16 - 1];  // clamped: no load under a branch
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      if (base + u * 256 < n16) acc ^= v[u];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] ^= red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

hipError_t launch_stream_read(const void* in, int64_t n16, uint32_t* out, int nblocks,
                              hipStream_t s) {
  if (n16 <= 0 || nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_read, dim3(nblocks), dim3(256), 0, s,
                     static_cast<const u32x4*>(in), n16, out);
  return hipGetLastError();
}

// Sticky status word: w[1] receives w[0], and w[0] is cleared, in one atomic
// exchange (stream-ordered after every clip kernel that ORed into w[0]).
__global__ void k_take_status(uint32_t* w) {
  if (threadIdx.x == 0) w[1] = atomicExch(w, 0u);
}

hipError_t launch_take_status(uint32_t* w, hipStream_t s) {
  hipLaunchKernelGGL(k_take_status, dim3(1), dim3(64), 0, s, w);
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
// span; this one is CholeskyQR (Gram matrix and its factor in fp64), repeated
// once on Q1 when Q1 is not yet orthonormal to fp32 precision (CholeskyQR2;
// ill-conditioned or rank-deficient sketches).  A pivot that vanishes
// relative to the largest diagonal entry zeroes its column of Q; the
// remaining columns still span range(X) and Q Q^T is the orthogonal
// projector onto it.  The vectors of length p are rows here (X^T's columns),
// split into chunks of kOrthChunk elements, one block per (chunk, sample);
// every reduction over p is a set of per-chunk fp64 partials that the next
// launch sums in chunk order.  Three launches:
//   k_orth_gram   X = the sum of the sketch's split partials; Gram(X) partials.
//   k_orth_first  R1 from Gram(X); Q1 = X R1^-1 (stored); partials of
//                 Gram(Q1) and H1 = Q1 W^T.
//   k_orth_final  R2 from Gram(Q1) (the identity when Gram(Q1) is within
//                 kOrthTol of I); Q = Q1 R2^-1; H = Q W^T = R2^-T H1;
//                 W' = W - H^T Q; writes [Q; W'] in fp32 or as zero-padded
//                 bf16 rows.
// Every step here is latency-bound (a few hundred KB per call), so the code
// is arranged around memory and LDS round trips: partial sums are loaded
// before the operands, the factorisation runs on one wave, and no global
// load sits under a condition.
// ---------------------------------------------------------------------------
constexpr int kOrthMaxCols = 32;
constexpr int kOrthChunk = 256;
constexpr int kOrthRow = kOrthChunk + 4;  // LDS row stride: 16-byte aligned, rows on distinct banks
constexpr double kOrthTol = 1e-7;  // |Gram(Q1) - I| entries below this skip the second factor

int orth_chunks(int p) { return (p + kOrthChunk - 1) / kOrthChunk; }
__host__ __device__ inline int orth_gram_pairs(int s) { return s * (s + 1) / 2; }  // packed upper triangle

__device__ __forceinline__ int packed_index(int i, int j) { return j * (j + 1) / 2 + i; }
__device__ __forceinline__ void unpack_index(int pi, int* i, int* j) {
  int c = 0;
  while ((c + 1) * (c + 2) / 2 <= pi) ++c;
  *j = c;
  *i = pi - c * (c + 1) / 2;
}

// sum_t a[t] b[t] over one chunk held in LDS; exact fp32 products, fp64 sums
// in four interleaved accumulators combined in a fixed order.
__device__ __forceinline__ double chunk_dot(const float* a, const float* b) {
  double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
#pragma unroll 4
  for (int t = 0; t < kOrthChunk; t += 4) {
    const float4 va = *reinterpret_cast<const float4*>(a + t);
    const float4 vb = *reinterpret_cast<const float4*>(b + t);
    acc0 = fma(static_cast<double>(va.x), static_cast<double>(vb.x), acc0);
    acc1 = fma(static_cast<double>(va.y), static_cast<double>(vb.y), acc1);
    acc2 = fma(static_cast<double>(va.z), static_cast<double>(vb.z), acc2);
    acc3 = fma(static_cast<double>(va.w), static_cast<double>(vb.w), acc3);
  }
  return (acc0 + acc1) + (acc2 + acc3);
}

// Sum of the chunk partials of one sample into LDS dst[npairs], each entry
// added up in chunk order, by a block of kOrthChunk threads (a constant: the
// block size read at run time is a memory load that would wait for every
// load issued before it).  The partials are contiguous ([chunk][pair]); tiles
// of whole chunks, kSumStage doubles at most, go through LDS.  The loads of
// the first tile are issued by partials_issue() so that a kernel can put them
// ahead of its operand loads: the memory counter drains in issue order, and
// waiting for the partials then does not wait for the operands.
constexpr int kSumStage = 4096;  // doubles of LDS staging, 16 per thread
constexpr int kSumPer = kSumStage / kOrthChunk;

__host__ __device__ inline int sum_tile_chunks(int npairs) {
  return npairs < kSumStage ? kSumStage / npairs : 1;
}

__device__ __forceinline__ void partials_issue(const double* part_b, int nchunk, int npairs,
                                               double (&v)[kSumPer]) {
  const int tile = sum_tile_chunks(npairs);
  const int n = (nchunk < tile ? nchunk : tile) * npairs;
#pragma unroll
  for (int k = 0; k < kSumPer; ++k) {  // clamped: no load under a condition
    const int u = k * kOrthChunk + threadIdx.x;
    v[k] = part_b[u < n ? u : n - 1];
  }
}

__device__ void partials_sum(const double* part_b, int nchunk, int npairs, double (&v)[kSumPer],
                             double* dst, double* stage) {
  const int tile = sum_tile_chunks(npairs);
  // first tile, straight-line: the stage holds exactly kSumPer values per
  // thread, so every store is in bounds (entries past the tile are not read)
  const int nc0 = nchunk < tile ? nchunk : tile;
#pragma unroll
  for (int k = 0; k < kSumPer; ++k) stage[k * kOrthChunk + threadIdx.x] = v[k];
  __syncthreads();
  for (int pi = threadIdx.x; pi < npairs; pi += kOrthChunk) {
    double acc = 0.0;
    for (int c = 0; c < nc0; ++c) acc += stage[c * npairs + pi];
    dst[pi] = acc;
  }
  for (int c0 = tile; c0 < nchunk; c0 += tile) {
    const int nc = nchunk - c0 < tile ? nchunk - c0 : tile;
    const int n = nc * npairs;
    const double* src = part_b + static_cast<int64_t>(c0) * npairs;
#pragma unroll
    for (int k = 0; k < kSumPer; ++k) {
      const int u = k * kOrthChunk + threadIdx.x;
      v[k] = src[u < n ? u : n - 1];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSumPer; ++k) stage[k * kOrthChunk + threadIdx.x] = v[k];
    __syncthreads();
    for (int pi = threadIdx.x; pi < npairs; pi += kOrthChunk) {
      double acc = dst[pi];
      for (int c = 0; c < nc; ++c) acc += stage[c * npairs + pi];
      dst[pi] = acc;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), lane));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), lane));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// 1/d and 1/sqrt(d) for normal d > 0: the hardware estimate and two Newton
// steps (each roughly doubles the correct bits), a few ulp from the rounded
// quotient and far shorter than the IEEE division sequence, which matters in
// the one-wave dependent chains below.
__device__ __forceinline__ double recip_f64(double d) {
  double r = __builtin_amdgcn_rcp(d);
  r = fma(fma(-d, r, 1.0), r, r);
  return fma(fma(-d, r, 1.0), r, r);
}
__device__ __forceinline__ double rsqrt_f64(double d) {
  double y = __builtin_amdgcn_rsq(d);
  y = fma(0.5 * y, fma(-d * y, y, 1.0), y);
  return fma(0.5 * y, fma(-d * y, y, 1.0), y);
}

// Inverse Cholesky factor of the s x s Gram matrix given as a packed upper
// triangle gp[packed_index(i, j)] (LDS).  Writes the transpose of R^-1,
// RinvT[j * S + i] = R^-1[i][j] (zero for i > j), with Gram = R^T R = L D L^T
// (L unit lower triangular), so R^-1 = L^-T D^-1/2.  A pivot not above 1e-24
// x the largest diagonal entry marks its column dead (zero row and column of
// R^-1).  Run by the first wave of the block; the caller synchronises after.
//   Elimination: lane i holds row i of the trailing matrix in registers.  At
//   step j lane j publishes its row in LDS (ws[0, S)) and every lane reads it
//   back as broadcasts.  The trailing block stays symmetric, so lane i's
//   multiplier L[i][j] = G[i][j] / d_j is entry i of the published row; it is
//   stored at ws[S + i * S + j].  Entries left of the pivot are not read again
//   and are left stale.  A wave executes its LDS operations in order, so the
//   publish and the reads need no barrier, only a compiler fence.
//   Inverse: lane c forms column c of L^-1 by forward substitution over the
//   stored multipliers, all columns at once.
// ws: LDS scratch of S * (S + 2) doubles.
template <int S>
__device__ __forceinline__ void inverse_cholesky_wave(const double* gp, int s, double* RinvT,
                                                      double* ws) {
  const int lane = threadIdx.x;
  double* prow = ws;              // [S] published pivot row
  double* Lm = ws + S;            // [S][S] multipliers
  double* rs = ws + S + S * S;    // [S] 1/sqrt(d_j), 0 when dead
  double g[S];
  double diag = 0.0;
#pragma unroll
  for (int c = 0; c < S; ++c) {
    const int i = lane < c ? lane : c, j = lane < c ? c : lane;
    g[c] = (lane < s && c < s) ? gp[packed_index(i, j)] : 0.0;
    diag = c == lane ? g[c] : diag;
  }
  if (lane < S) prow[lane] = diag;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  double dmax = 0.0;
#pragma unroll
  for (int c = 0; c < S; ++c) dmax = fmax(dmax, prow[c]);  // zero beyond s
  const double tiny = dmax * 1e-24;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const int me = lane < S ? lane : S - 1;
  double piv = 0.0;  // lane j: its pivot, 0 when dead
  const double2* prow2 = reinterpret_cast<const double2*>(prow);
#pragma unroll 1
  for (int j = 0; j < s; ++j) {
    if (lane == j) {
#pragma unroll
      for (int c = 0; c < S; c += 2) reinterpret_cast<double2*>(prow)[c / 2] = make_double2(g[c], g[c + 1]);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const double dj = prow[j];
    const double gi = prow[me];
    double pr[S];
#pragma unroll
    for (int c = 0; c < S; c += 2) {
      const double2 v = prow2[c / 2];
      pr[c] = v.x;
      pr[c + 1] = v.y;
    }
    const bool live = dj > tiny;
    const double f = (live && lane > j && lane < s) ? gi * recip_f64(dj) : 0.0;
    if (lane == j) piv = live ? dj : 0.0;
    if (lane < S) Lm[lane * S + j] = f;
#pragma unroll
    for (int c = 0; c < S; ++c) g[c] = fma(-f, pr[c], g[c]);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  if (lane < S) rs[lane] = piv > 0.0 ? rsqrt_f64(piv) : 0.0;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  // column c = lane of L^-1: y_c = 1, y_i = -sum_{c <= k < i} L[i][k] y_k (i > c)
  double y[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < i; ++k) acc = fma(-Lm[i * S + k], y[k], acc);
    y[i] = i == lane ? 1.0 : (i > lane && i < s ? acc : 0.0);
  }
  // R^-1[c][i] = L^-1[i][c] / sqrt(d_i), stored as RinvT[i][c]
  if (lane < S) {
#pragma unroll
    for (int i = 0; i < S; ++i) RinvT[i * S + lane] = lane < s ? y[i] * rs[i] : 0.0;
  }
}

// y[j] = sum_{i <= j} x[i] R^-1[i][j] for j < s (zero beyond), fp64, reading
// row j of RinvT with 16-byte LDS loads; terms in ascending i.
template <int S>
__device__ __forceinline__ void apply_rinv(const float (&x)[S], const double* RinvT, int s,
                                           double (&y)[S]) {
#pragma unroll
  for (int j = 0; j < S; ++j) {
    double acc = 0.0;
    if (j < s) {
      const double2* row = reinterpret_cast<const double2*>(RinvT + j * S);
#pragma unroll
      for (int i2 = 0; 2 * i2 <= j; ++i2) {
        const double2 rv = row[i2];
        acc = fma(static_cast<double>(x[2 * i2]), rv.x, acc);
        if (2 * i2 + 1 <= j) acc = fma(static_cast<double>(x[2 * i2 + 1]), rv.y, acc);
      }
    }
    y[j] = acc;
  }
}

// Global loads below are unconditional from clamped (always valid) addresses,
// with out-of-range values replaced afterwards: a load under a condition
// makes the compiler wait for it before the branch joins, which serialises
// the whole batch of row loads into one memory latency each.

// v[i] = rows[i][e] for i < nrows and e < p, else 0 (nrows >= 1, p >= 1).
template <int N>
__device__ __forceinline__ void load_rows(const float* base, int nrows, int p, int e,
                                          float (&v)[N]) {
  const int ec = e < p ? e : p - 1;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = base[static_cast<int64_t>(i < nrows ? i : nrows - 1) * p + ec];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = (i < nrows && e < p) ? v[i] : 0.f;
}

// Marks values as used at this point: arithmetic on them cannot be hoisted
// above it, so waiting for the loads that produced them happens here.
template <int N>
__device__ __forceinline__ void use_here(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// The sketch is the sum of the projection's split partials: x[i] = sum_sp
// X[b][sp][i][e] (i < s), added in split order.  sketch_issue() loads splits
// 0 and 1 (split 0 twice when there is one); sketch_finish() adds them and
// any further splits.
template <int S>
__device__ __forceinline__ void sketch_issue(const float* xb, int nsplit, int64_t split_stride,
                                             int s, int p, int e, float (&v0)[S], float (&v1)[S]) {
  load_rows<S>(xb, s, p, e, v0);
  load_rows<S>(xb + (nsplit > 1 ? split_stride : 0), s, p, e, v1);
}

template <int S>
__device__ __forceinline__ void sketch_finish(const float* xb, int nsplit, int64_t split_stride,
                                              int s, int p, int e, const float (&v0)[S],
                                              const float (&v1)[S], float (&x)[S]) {
#pragma unroll
  for (int i = 0; i < S; ++i) x[i] = nsplit > 1 ? v0[i] + v1[i] : v0[i];
  for (int sp = 2; sp < nsplit; ++sp) {
    float v[S];
    load_rows<S>(xb + sp * split_stride, s, p, e, v);
#pragma unroll
    for (int i = 0; i < S; ++i) x[i] += v[i];
  }
}

// part1[b][chunk][packed (i, j)] = sum_{e in chunk} X[i][e] X[j][e].
template <int S>
__global__ void __launch_bounds__(kOrthChunk) k_orth_gram(
    const float* __restrict__ Xp, int nsplit, int64_t split_stride, int64_t x_bstride, int s,
    int p, double* __restrict__ part1) {
  __shared__ __align__(16) float rows[S][kOrthRow];
  const int b = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int e = chunk * kOrthChunk + tid;
  const float* xb = Xp + b * x_bstride;
  float x0[S], x1[S], x[S];
  sketch_issue<S>(xb, nsplit, split_stride, s, p, e, x0, x1);
  sketch_finish<S>(xb, nsplit, split_stride, s, p, e, x0, x1, x);
#pragma unroll
  for (int i = 0; i < S; ++i)
    if (i < s) rows[i][tid] = x[i];
  __syncthreads();
  const int np = orth_gram_pairs(s);
  double* out = part1 + (static_cast<int64_t>(b) * gridDim.x + chunk) * np;
  for (int pi = tid; pi < np; pi += kOrthChunk) {
    int i, j;
    unpack_index(pi, &i, &j);
    out[pi] = chunk_dot(rows[i], rows[j]);
  }
}

// Q1 = X R1^-1 into Q1 rows 0..s-1; part2[b][chunk][.] = packed Gram(Q1)
// partials, then H1[i][t] = sum_e Q1[i][e] W[t][e] at packed_pairs + i * r + t.
// S, R: the largest s and r the instance handles.
template <int S, int R>
__global__ void __launch_bounds__(kOrthChunk) k_orth_first(
    const float* __restrict__ Xp, int nsplit, int64_t split_stride, int64_t x_bstride, int s,
    int p, const double* __restrict__ part1, const float* __restrict__ W, int64_t w_bstride, int r,
    float* __restrict__ Q1, int64_t q_bstride, double* __restrict__ part2) {
  __shared__ double stage[kSumStage];
  __shared__ double gp[S * (S + 1) / 2];
  __shared__ __align__(16) double RinvT[S * S];
  __shared__ __align__(16) double chol_ws[S * (S + 2)];
  __shared__ __align__(16) float rows[S + R][kOrthRow];
  const int b = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x, nch = gridDim.x;
  const int e = chunk * kOrthChunk + tid;
  // partials first, then the operands: their latency overlaps the partial
  // sums and the factorisation
  const int np1 = orth_gram_pairs(s);
  const double* pb = part1 + static_cast<int64_t>(b) * nch * np1;
  double pv[kSumPer];
  partials_issue(pb, nch, np1, pv);
  const float* xb = Xp + b * x_bstride;
  float x0[S], x1[S], x[S], w[R];
  sketch_issue<S>(xb, nsplit, split_stride, s, p, e, x0, x1);
  load_rows<R>(W + b * w_bstride, r, p, e, w);
  partials_sum(pb, nch, np1, pv, gp, stage);
  if (tid < 64) inverse_cholesky_wave<S>(gp, s, RinvT, chol_ws);
  __syncthreads();
  use_here<S>(x0);
  use_here<S>(x1);
  use_here<R>(w);
  sketch_finish<S>(xb, nsplit, split_stride, s, p, e, x0, x1, x);
  float* qb = Q1 + b * q_bstride;
  double q[S];
  apply_rinv<S>(x, RinvT, s, q);
#pragma unroll
  for (int j = 0; j < S; ++j) {
    if (j < s) {
      const float qf = e < p ? static_cast<float>(q[j]) : 0.f;
      rows[j][tid] = qf;
      if (e < p) qb[static_cast<int64_t>(j) * p + e] = qf;
    }
  }
#pragma unroll
  for (int t = 0; t < R; ++t)
    if (t < r) rows[S + t][tid] = w[t];
  __syncthreads();
  const int np2 = np1 + s * r;
  double* out = part2 + (static_cast<int64_t>(b) * nch + chunk) * np2;
  for (int pi = tid; pi < np2; pi += kOrthChunk) {
    int i, j;
    if (pi < np1) {
      unpack_index(pi, &i, &j);
    } else {
      i = (pi - np1) / r;
      j = S + (pi - np1) % r;
    }
    out[pi] = chunk_dot(rows[i], rows[j]);
  }
}

// Q = Q1 R2^-1, H = R2^-T H1, W' = W - H^T Q; rows 0..s-1 = Q, s..s+r-1 = W',
// then zero rows up to out_rows.  TOut float: in place over Q1's buffer is
// allowed (every thread reads its own elements before writing them).
template <int S, int R, typename TOut>
__global__ void __launch_bounds__(kOrthChunk) k_orth_final(
    const float* Q1, int64_t q_bstride, int s, int p, const double* __restrict__ part2,
    const float* __restrict__ W, int64_t w_bstride, int r, TOut* out, int64_t o_bstride,
    int out_rows) {
  __shared__ double stage[kSumStage];
  __shared__ double gh[S * (S + 1) / 2 + S * R];
  __shared__ __align__(16) double RinvT[S * S];
  __shared__ __align__(16) double chol_ws[S * (S + 2)];
  __shared__ __align__(16) double HT[R * S];  // HT[t * S + j] = H[j][t]
  const int b = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x, nch = gridDim.x;
  const int e = chunk * kOrthChunk + tid;
  const int np1 = orth_gram_pairs(s);
  const int np2 = np1 + s * r;
  const double* pb = part2 + static_cast<int64_t>(b) * nch * np2;
  double pv[kSumPer];
  partials_issue(pb, nch, np2, pv);
  float q1[S], w[R];
  load_rows<S>(Q1 + b * q_bstride, s, p, e, q1);
  load_rows<R>(W + b * w_bstride, r, p, e, w);
  partials_sum(pb, nch, np2, pv, gh, stage);
  // When Gram(Q1) is within kOrthTol of I, Q1 is already orthonormal to fp32
  // precision (the precision Q is stored in), and the second factor is the
  // identity; otherwise (ill-conditioned or rank-deficient sketches) factor it.
  bool far = false;
  for (int pi = tid; pi < np1; pi += kOrthChunk) {
    int i, j;
    unpack_index(pi, &i, &j);
    far |= !(fabs(gh[pi] - (i == j ? 1.0 : 0.0)) <= kOrthTol);
  }
  if (__syncthreads_or(far)) {
    if (tid < 64) inverse_cholesky_wave<S>(gh, s, RinvT, chol_ws);
  } else {
    for (int u = tid; u < S * S; u += kOrthChunk)
      RinvT[u] = (u / S == u % S && u % S < s) ? 1.0 : 0.0;
  }
  __syncthreads();
  // H[j][t] = sum_{i <= j} R2^-1[i][j] H1[i][t]
  for (int u = tid; u < s * r; u += kOrthChunk) {
    const int j = u / r, t = u % r;
    double h = 0.0;
    for (int i = 0; i <= j; ++i) h = fma(RinvT[j * S + i], gh[np1 + i * r + t], h);
    HT[t * S + j] = h;
  }
  const int nz = S - s;  // rows t < r are read in full: zero their entries j >= s
  for (int u = tid; u < r * nz; u += kOrthChunk) HT[(u / nz) * S + s + u % nz] = 0.0;
  __syncthreads();
  use_here<S>(q1);
  use_here<R>(w);
  if (e >= p) return;
  double qd[S];
  apply_rinv<S>(q1, RinvT, s, qd);
  float q[S];
#pragma unroll
  for (int j = 0; j < S; ++j) q[j] = static_cast<float>(qd[j]);
  TOut* ob = out + b * o_bstride;
#pragma unroll
  for (int j = 0; j < S; ++j)
    if (j < s) ob[static_cast<int64_t>(j) * p + e] = to_out<TOut>(q[j]);
#pragma unroll
  for (int t = 0; t < R; ++t) {
    if (t < r) {
      const double2* row = reinterpret_cast<const double2*>(HT + t * S);
      double v = w[t];
#pragma unroll
      for (int j2 = 0; j2 < S / 2; ++j2) {
        const double2 hv = row[j2];
        v = fma(-hv.x, static_cast<double>(q[2 * j2]), v);
        v = fma(-hv.y, static_cast<double>(q[2 * j2 + 1]), v);
      }
      ob[static_cast<int64_t>(s + t) * p + e] = to_out<TOut>(static_cast<float>(v));
    }
  }
  for (int row = s + r; row < out_rows; ++row) ob[static_cast<int64_t>(row) * p + e] = to_out<TOut>(0.f);
}

size_t hpp_orth_scratch_bytes(int B, int p, int s, int r) {
  const int np1 = orth_gram_pairs(s), np2 = np1 + s * r;
  return static_cast<size_t>(B) * orth_chunks(p) * (np1 + np2) * sizeof(double);
}

template <int S, int R>
static hipError_t orth_launch(const float* Xp, int nsplit, int64_t split_stride,
                              int64_t x_bstride, const float* W, int64_t w_bstride, int B, int p,
                              int s, int r, float* P3, bf16_t* P3b, int p3b_rows, double* scratch,
                              hipStream_t st) {
  const int nch = orth_chunks(p);
  const dim3 grid(nch, B);
  double* part1 = scratch;
  double* part2 = scratch + static_cast<int64_t>(B) * nch * orth_gram_pairs(s);
  const int64_t p3s = static_cast<int64_t>(s + r) * p;
  hipLaunchKernelGGL(k_orth_gram<S>, grid, dim3(kOrthChunk), 0, st, Xp, nsplit, split_stride,
                     x_bstride, s, p, part1);
  hipLaunchKernelGGL((k_orth_first<S, R>), grid, dim3(kOrthChunk), 0, st, Xp, nsplit,
                     split_stride, x_bstride, s, p, part1, W, w_bstride, r, P3, p3s, part2);
  if (P3b) {
    hipLaunchKernelGGL((k_orth_final<S, R, bf16_t>), grid, dim3(kOrthChunk), 0, st, P3, p3s, s,
                       p, part2, W, w_bstride, r, P3b, static_cast<int64_t>(p3b_rows) * p,
                       p3b_rows);
  } else {
    hipLaunchKernelGGL((k_orth_final<S, R, float>), grid, dim3(kOrthChunk), 0, st, P3, p3s, s, p,
                       part2, W, w_bstride, r, P3, p3s, s + r);
  }
  return hipGetLastError();
}

hipError_t launch_hpp_orth(const float* Xp, int nsplit, int64_t split_stride, int64_t x_bstride,
                           const float* W, int64_t w_bstride, int B, int p, int s, int r,
                           float* P3, bf16_t* P3b, int p3b_rows, double* scratch, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (s < 1 || s > kOrthMaxCols || r < 1 || r > kOrthMaxCols || nsplit < 1 || p < 1)
    return hipErrorInvalidValue;
  if (P3b && p3b_rows < s + r) return hipErrorInvalidValue;
#define DPRC_ORTH(SS, RR)                                                                       \
  return orth_launch<SS, RR>(Xp, nsplit, split_stride, x_bstride, W, w_bstride, B, p, s, r, P3, \
                             P3b, p3b_rows, scratch, st)
  if (s <= 16) {
    if (r <= 16) DPRC_ORTH(16, 16);
    DPRC_ORTH(16, 32);
  }
  if (r <= 16) DPRC_ORTH(32, 16);
  DPRC_ORTH(32, 32);
#undef DPRC_ORTH
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
