// Random streams of the method on gfx950: Hutchinson probes and DP noise from
// Philox4x32-10 + Box-Muller, and the fused noise-add + SGD update.
//
// Probe entry (row r, column j) of sample i in layer l is lane r mod 4 of the
// counter (r / 4, j, i, l) under key `seed` (the randomized-clipping summary,
// section 中核メカニズム, item 1: P has i.i.d. Gaussian entries).  The noise of
// flat parameter index e is lane e mod 4 of (lo(e / 4), hi(e / 4), 0xFFFFFFFF, l)
// (glossary page, section DP-SGDのアルゴリズム, step 4).
#include "common.h"
#include "internal.h"

namespace dprc {

__global__ void k_philox_u32(uint32_t k0, uint32_t k1, const uint32_t* __restrict__ ctr,
                             uint32_t* __restrict__ out, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u32x4 c;
  c.x = ctr[4 * i + 0];
  c.y = ctr[4 * i + 1];
  c.z = ctr[4 * i + 2];
  c.w = ctr[4 * i + 3];
  const u32x4 w = philox4x32_10(c, k0, k1);
  out[4 * i + 0] = w.x;
  out[4 * i + 1] = w.y;
  out[4 * i + 2] = w.z;
  out[4 * i + 3] = w.w;
}

hipError_t launch_philox_u32(uint64_t seed, const uint32_t* ctr, uint32_t* out, size_t n,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(k_philox_u32, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t>(seed),
                     static_cast<uint32_t>(seed >> 32), ctr, out, n);
  return hipGetLastError();
}

// One thread per (sample, column j, row group g): four rows 4g..4g+3 of column j.
// signs != 0: Rademacher entries, +1 when the counter word's top bit is 0 and
// -1 otherwise (summary, section 意義と主張: {+-1}-valued sketching matrices).
template <typename TOut>
__global__ void k_probe_fill(uint32_t k0, uint32_t k1, uint32_t layer, uint32_t sample0, int p,
                             int kfill, int kpad, TOut* __restrict__ out,
                             int signs) {
  const int ngroups = (p + 3) >> 2;
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  const int j = blockIdx.y;
  const int i = blockIdx.z;
  if (g >= ngroups) return;
  float z[4] = {0.f, 0.f, 0.f, 0.f};
  if (j < kfill) {
    u32x4 c;
    c.x = static_cast<uint32_t>(g);
    c.y = static_cast<uint32_t>(j);
    c.z = sample0 + static_cast<uint32_t>(i);
    c.w = layer;
    if (signs) {
      const u32x4 w = philox4x32_10(c, k0, k1);
#pragma unroll
      for (int l = 0; l < 4; ++l) z[l] = (w[l] >> 31) ? -1.f : 1.f;
    } else {
      normals4(c, k0, k1, z);
    }
  }
  TOut* row = out + (static_cast<int64_t>(i) * kpad + j) * p;
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    const int r = 4 * g + l;
    if (r < p) {
      if constexpr (sizeof(TOut) == 4)
        row[r] = z[l];
      else
        row[r] = f32_to_bf16(z[l]);
    }
  }
}

template <typename TOut>
static hipError_t probe_fill(uint64_t seed, uint32_t layer, uint32_t sample0, int nsamp, int p,
                             int kfill, int kpad, TOut* out, hipStream_t s, bool signs) {
  if (nsamp <= 0 || p <= 0 || kpad <= 0) return hipSuccess;
  const int ngroups = (p + 3) >> 2;
  dim3 grid((ngroups + 255) / 256, kpad, nsamp);
  hipLaunchKernelGGL(k_probe_fill<TOut>, grid, dim3(256), 0, s, static_cast<uint32_t>(seed),
                     static_cast<uint32_t>(seed >> 32), layer, sample0, p, kfill, kpad, out,
                     signs ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_probe_fill_f32(uint64_t seed, uint32_t layer, uint32_t sample0, int nsamp,
                                 int p, int kfill, int kpad, float* out, hipStream_t s,
                                 bool signs) {
  return probe_fill<float>(seed, layer, sample0, nsamp, p, kfill, kpad, out, s, signs);
}

hipError_t launch_probe_fill_bf16(uint64_t seed, uint32_t layer, uint32_t sample0, int nsamp,
                                  int p, int kfill, int kpad, bf16_t* out, hipStream_t s,
                                  bool signs) {
  return probe_fill<bf16_t>(seed, layer, sample0, nsamp, p, kfill, kpad, out, s, signs);
}

// Probes of up to kProbeLayersMax layers in one launch, bf16, padded to kpad
// columns: the same entries as k_probe_fill for each layer.  Workgroup x walks
// the layers' row-group blocks in order (layer t owns blocks bstart[t] ..
// bstart[t + 1] - 1), z is the sample, and each thread fills its four rows in
// the columns of range y (jper columns) in turn: with many layers one range
// covers every column, one workgroup per 1024 rows and sample instead of one
// per column as well, since workgroups that each write only 2 KB are limited
// by how fast they can be dispatched; a launch of few layers splits the
// columns so that the chip still gets about a thousand workgroups.
template <int N>
__global__ void k_probe_fill_layers(uint32_t k0, uint32_t k1, ProbeLayerTable<N> tab, int kfill,
                                    int kpad, int jper, bf16_t* __restrict__ out, int signs) {
  int t = 0;
  while (t + 1 < tab.n && static_cast<int>(blockIdx.x) >= tab.bstart[t + 1]) ++t;
  const int p = tab.p[t];
  const int ngroups = (p + 3) >> 2;
  const int g = (static_cast<int>(blockIdx.x) - tab.bstart[t]) * blockDim.x + threadIdx.x;
  const int i = blockIdx.z;
  if (g >= ngroups) return;
  bf16_t* base = out + tab.off[t] + static_cast<int64_t>(i) * kpad * p;
  const int j0 = static_cast<int>(blockIdx.y) * jper;
  const int j1 = j0 + jper < kpad ? j0 + jper : kpad;
  for (int j = j0; j < j1; ++j) {
    float z[4] = {0.f, 0.f, 0.f, 0.f};
    if (j < kfill) {
      u32x4 c;
      c.x = static_cast<uint32_t>(g);
      c.y = static_cast<uint32_t>(j);
      c.z = static_cast<uint32_t>(i);
      c.w = tab.layer[t];
      if (signs) {
        const u32x4 w = philox4x32_10(c, k0, k1);
#pragma unroll
        for (int l = 0; l < 4; ++l) z[l] = (w[l] >> 31) ? -1.f : 1.f;
      } else {
        normals4(c, k0, k1, z);
      }
    }
    bf16_t* row = base + static_cast<int64_t>(j) * p;
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int r = 4 * g + l;
      if (r < p) row[r] = f32_to_bf16(z[l]);
    }
  }
}

hipError_t launch_probe_fill_layers_bf16(uint64_t seed, const ProbeLayerTable<kProbeLayersMax>& tab,
                                         int nsamp, int kfill, int kpad, bf16_t* out,
                                         hipStream_t s, bool signs) {
  if (nsamp <= 0 || kpad <= 0 || tab.n <= 0) return hipSuccess;
  if (tab.n > kProbeLayersMax) return hipErrorInvalidValue;
  const int nblocks = tab.bstart[tab.n];
  if (nblocks <= 0) return hipSuccess;
  // column ranges: enough for about 1024 workgroups, at most one column each
  const int64_t wgs = static_cast<int64_t>(nblocks) * nsamp;
  int64_t want = (1024 + wgs - 1) / wgs;
  if (want > kpad) want = kpad;
  const int jper = static_cast<int>((kpad + want - 1) / want);
  const int nrange = (kpad + jper - 1) / jper;
  hipLaunchKernelGGL(k_probe_fill_layers<kProbeLayersMax>, dim3(nblocks, nrange, nsamp), dim3(256), 0,
                     s, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), tab, kfill,
                     kpad, jper, out, signs ? 1 : 0);
  return hipGetLastError();
}

// xi[e - offset] for e in [offset, offset + n); one thread per counter group.
__global__ void k_noise_fill(uint32_t k0, uint32_t k1, uint32_t layer, uint64_t offset, size_t n,
                             float* __restrict__ xi) {
  const uint64_t g0 = offset >> 2;
  const uint64_t g = g0 + static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const uint64_t end = offset + n;
  if ((g << 2) >= end) return;
  float z[4];
  normals4(noise_counter(g, layer), k0, k1, z);
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    const uint64_t e = (g << 2) + l;
    if (e >= offset && e < end) xi[e - offset] = z[l];
  }
}

hipError_t launch_noise_fill(uint64_t seed, uint32_t layer, uint64_t offset, size_t n, float* xi,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint64_t groups = ((offset + n + 3) >> 2) - (offset >> 2);
  hipLaunchKernelGGL(k_noise_fill, dim3(static_cast<unsigned>((groups + 255) / 256)), dim3(256), 0,
                     s, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), layer,
                     offset, n, xi);
  return hipGetLastError();
}

// theta[e] -= eta_over_B * (S[e] + sigmaC * xi[e]) for four consecutive e per
// thread (one Philox block); 16-byte vector accesses when the group is whole.
__global__ void __launch_bounds__(256) k_noise_update(float* __restrict__ theta,
                                                      const float* __restrict__ S, int64_t n,
                                                      float sigmaC, float eta_over_B, uint32_t k0,
                                                      uint32_t k1, uint32_t layer) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t e0 = g << 2;
  if (e0 >= n) return;
  float z[4];
  normals4(noise_counter(static_cast<uint64_t>(g), layer), k0, k1, z);
  if (e0 + 3 < n) {
    float4 th = *reinterpret_cast<const float4*>(theta + e0);
    const float4 sv = *reinterpret_cast<const float4*>(S + e0);
    th.x -= eta_over_B * fmaf(sigmaC, z[0], sv.x);
    th.y -= eta_over_B * fmaf(sigmaC, z[1], sv.y);
    th.z -= eta_over_B * fmaf(sigmaC, z[2], sv.z);
    th.w -= eta_over_B * fmaf(sigmaC, z[3], sv.w);
    *reinterpret_cast<float4*>(theta + e0) = th;
  } else {
    for (int l = 0; l < 4 && e0 + l < n; ++l)
      theta[e0 + l] -= eta_over_B * fmaf(sigmaC, z[l], S[e0 + l]);
  }
}

// The same update with S = sum over nsplit planes part[split][e] formed on the
// fly (split order, as the separate reduction), optionally stored to S_out.
__global__ void __launch_bounds__(256) k_noise_update_splits(float* __restrict__ theta,
                                                             const float* __restrict__ part,
                                                             int nsplit, int64_t n,
                                                             float* __restrict__ S_out,
                                                             float sigmaC, float eta_over_B,
                                                             uint32_t k0, uint32_t k1,
                                                             uint32_t layer) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t e0 = g << 2;
  if (e0 >= n) return;
  float z[4];
  normals4(noise_counter(static_cast<uint64_t>(g), layer), k0, k1, z);
  if (e0 + 3 < n) {
    float4 sv = *reinterpret_cast<const float4*>(part + e0);
    for (int sp = 1; sp < nsplit; ++sp) {
      const float4 v = *reinterpret_cast<const float4*>(part + sp * n + e0);
      sv.x += v.x;
      sv.y += v.y;
      sv.z += v.z;
      sv.w += v.w;
    }
    if (S_out) *reinterpret_cast<float4*>(S_out + e0) = sv;
    float4 th = *reinterpret_cast<const float4*>(theta + e0);
    th.x -= eta_over_B * fmaf(sigmaC, z[0], sv.x);
    th.y -= eta_over_B * fmaf(sigmaC, z[1], sv.y);
    th.z -= eta_over_B * fmaf(sigmaC, z[2], sv.z);
    th.w -= eta_over_B * fmaf(sigmaC, z[3], sv.w);
    *reinterpret_cast<float4*>(theta + e0) = th;
  } else {
    for (int l = 0; l < 4 && e0 + l < n; ++l) {
      float acc = 0.f;
      for (int sp = 0; sp < nsplit; ++sp) acc += part[sp * n + e0 + l];
      if (S_out) S_out[e0 + l] = acc;
      theta[e0 + l] -= eta_over_B * fmaf(sigmaC, z[l], acc);
    }
  }
}

hipError_t launch_noise_update_splits(float* theta, const float* part, int nsplit, int64_t n,
                                      float* S_out, float sigmaC, float eta_over_B, uint64_t seed,
                                      uint32_t layer, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t groups = (n + 3) >> 2;
  hipLaunchKernelGGL(k_noise_update_splits, dim3(static_cast<unsigned>((groups + 255) / 256)),
                     dim3(256), 0, s, theta, part, nsplit, n, S_out, sigmaC, eta_over_B,
                     static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), layer);
  return hipGetLastError();
}

hipError_t launch_noise_update(float* theta, const float* S, int64_t n, float sigmaC,
                               float eta_over_B, uint64_t seed, uint32_t layer, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t groups = (n + 3) >> 2;
  hipLaunchKernelGGL(k_noise_update, dim3(static_cast<unsigned>((groups + 255) / 256)), dim3(256),
                     0, s, theta, S, n, sigmaC, eta_over_B, static_cast<uint32_t>(seed),
                     static_cast<uint32_t>(seed >> 32), layer);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Poisson subsampling of the minibatch (glossary page, section
// DP-SGDのアルゴリズム, step 1: every example is in independently with
// probability q).  Example n of N is in step `step`'s minibatch when word
// n mod 4 of the counter (lo(n / 4), hi(n / 4), step, kPoissonC3) is below
// thr = floor(q 2^32): an integer comparison, exact on any device.  The
// indices come out in ascending order: per tile of kPoisTile examples a
// count, one exclusive scan of the counts, then every tile recomputes its
// draws and writes them at its offset (three launches, deterministic).
// ---------------------------------------------------------------------------
constexpr uint32_t kPoissonC3 = 0xFFFFFFFEu;
constexpr int kPoisThreads = 256;
constexpr int kPoisPer = 16;                        // examples per thread: four counters
constexpr int kPoisTile = kPoisThreads * kPoisPer;  // examples per block
constexpr int kScanThreads = 1024;

// Membership bits of examples e0 .. e0 + 15 (e0 a multiple of 16).
__device__ __forceinline__ uint32_t poisson_bits(uint32_t k0, uint32_t k1, uint32_t step,
                                                 uint64_t thr, int64_t e0, int64_t N) {
  uint32_t bits = 0;
  const uint64_t g0 = static_cast<uint64_t>(e0) >> 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t g = g0 + j;
    u32x4 c;
    c.x = static_cast<uint32_t>(g);
    c.y = static_cast<uint32_t>(g >> 32);
    c.z = step;
    c.w = kPoissonC3;
    const u32x4 w = philox4x32_10(c, k0, k1);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const bool in = e0 + 4 * j + l < N && static_cast<uint64_t>(ws[l]) < thr;
      bits |= (in ? 1u : 0u) << (4 * j + l);
    }
  }
  return bits;
}

// Exclusive prefix sum over the block (blockDim.x == NT, a multiple of 64);
// *total gets the block total.  red: LDS of NT / 64 values.
template <typename T, int NT>
__device__ __forceinline__ T block_exclusive_scan(T v, T* red, T* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) red[wid] = x;
  __syncthreads();
  T before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    before += w < wid ? red[w] : T(0);
    tot += red[w];
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

__global__ void __launch_bounds__(kPoisThreads) k_poisson_count(uint32_t k0, uint32_t k1,
                                                                uint32_t step, uint64_t thr,
                                                                int64_t N,
                                                                int64_t* __restrict__ counts) {
  __shared__ int red[kPoisThreads / 64];
  const int64_t e0 = static_cast<int64_t>(blockIdx.x) * kPoisTile + threadIdx.x * kPoisPer;
  const int c = __popc(poisson_bits(k0, k1, step, thr, e0, N));
  int total;
  block_exclusive_scan<int, kPoisThreads>(c, red, &total);
  if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

// One block: counts[0, nblk) -> exclusive offsets in place; *count = sum.
__global__ void __launch_bounds__(kScanThreads) k_poisson_scan(int64_t* __restrict__ counts,
                                                              int64_t nblk,
                                                              int64_t* __restrict__ count) {
  __shared__ int64_t red[kScanThreads / 64];
  int64_t carry = 0;
  for (int64_t b0 = 0; b0 < nblk; b0 += kScanThreads) {
    const int64_t b = b0 + threadIdx.x;
    const int64_t v = b < nblk ? counts[b] : 0;
    int64_t total;
    const int64_t ex = block_exclusive_scan<int64_t, kScanThreads>(v, red, &total);
    if (b < nblk) counts[b] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) *count = carry;
}

__global__ void __launch_bounds__(kPoisThreads) k_poisson_write(
    uint32_t k0, uint32_t k1, uint32_t step, uint64_t thr, int64_t N,
    const int64_t* __restrict__ offsets, int64_t* __restrict__ idx, int64_t cap) {
  __shared__ int red[kPoisThreads / 64];
  const int64_t e0 = static_cast<int64_t>(blockIdx.x) * kPoisTile + threadIdx.x * kPoisPer;
  const uint32_t bits = poisson_bits(k0, k1, step, thr, e0, N);
  int total;
  const int ex = block_exclusive_scan<int, kPoisThreads>(__popc(bits), red, &total);
  int64_t pos = offsets[blockIdx.x] + ex;
#pragma unroll
  for (int j = 0; j < kPoisPer; ++j) {
    if (bits >> j & 1u) {
      if (pos < cap) idx[pos] = e0 + j;
      ++pos;
    }
  }
}

int64_t poisson_blocks(int64_t N) { return (N + kPoisTile - 1) / kPoisTile; }

hipError_t launch_poisson_sample(uint64_t seed, uint32_t step, int64_t N, uint64_t thr,
                                 int64_t* idx, int64_t cap, int64_t* count, int64_t* counts,
                                 hipStream_t s) {
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  const int64_t nblk = poisson_blocks(N);
  if (nblk > 0)
    hipLaunchKernelGGL(k_poisson_count, dim3(static_cast<unsigned>(nblk)), dim3(kPoisThreads), 0,
                       s, k0, k1, step, thr, N, counts);
  hipLaunchKernelGGL(k_poisson_scan, dim3(1), dim3(kScanThreads), 0, s, counts, nblk, count);
  if (nblk > 0 && cap > 0)
    hipLaunchKernelGGL(k_poisson_write, dim3(static_cast<unsigned>(nblk)), dim3(kPoisThreads), 0,
                       s, k0, k1, step, thr, N, counts, idx, cap);
  return hipGetLastError();
}

}  // namespace dprc
