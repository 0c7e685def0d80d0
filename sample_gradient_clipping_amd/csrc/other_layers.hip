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

namespace dprc {

// ---------------------------------------------------------------------------
// Embedding table (h_t = E[id_t]): sample i's gradient in E has row v equal to
// the sum of delta_{i,t} over the tokens with id_t = v, so its squared norm is
// the sum over the distinct ids of the squared row norms.  Per sample the
// (id, position) pairs are sorted in LDS (bitonic, T <= kEmbMaxT); equal ids
// then form contiguous groups.  The norm pass streams the delta rows in sorted
// order, one block per (2048-column chunk, split, sample), where every split
// is a run of whole groups (no group crosses a block); the table update looks
// each row up in a per-sample row map and adds the dense noise.
// ---------------------------------------------------------------------------
constexpr int kEmbMaxT = 16384;
constexpr int kEmbSortThreads = 1024;

// spos, sid: sorted token positions and their ids; gidp: group index of each
// sorted position; ustart[g]: first sorted position of group g (ustart[ng] =
// T); uid[g]: its id; ng: number of groups.
//
// Bitonic sort of N = 1024 E keys (id << 32 | position, padded with ~0) in a
// blocked layout: thread t holds keys t E .. t E + E - 1 in registers.  A
// compare-exchange at distance j < E stays in the thread, at E <= j < 64 E it
// is a shuffle within the wave, and only the wider ones go through LDS.
template <int E>
__global__ void __launch_bounds__(kEmbSortThreads) k_emb_sort(
    const int32_t* __restrict__ ids, int T, int32_t* __restrict__ spos,
    int32_t* __restrict__ sid, int32_t* __restrict__ gidp, int32_t* __restrict__ ustart,
    int32_t* __restrict__ uid, int32_t* __restrict__ ng) {
  constexpr int N = kEmbSortThreads * E;
  __shared__ uint64_t xch[N];
  __shared__ int red[kEmbSortThreads / 64];
  __shared__ uint64_t wave_last[kEmbSortThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int32_t* ib = ids + static_cast<int64_t>(b) * T;
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = tid * E + e;
    const int jc = j < T ? j : T - 1;  // clamped, then replaced: no load under a condition
    const uint64_t key =
        (static_cast<uint64_t>(static_cast<uint32_t>(ib[jc])) << 32) | static_cast<uint32_t>(j);
    x[e] = j < T ? key : ~0ull;
  }
  for (int k = 2; k <= N; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int pe = e ^ jj;
          if (pe > e) {
            const int i = tid * E + e;
            const bool up = (i & k) == 0;
            const uint64_t a = x[e], c = x[pe];
            if ((a > c) == up) {
              x[e] = c;
              x[pe] = a;
            }
          }
        }
      } else if (jj < 64 * E) {
        const int dl = jj / E;  // partner lane distance
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = tid * E + e;
          const uint64_t other = __shfl_xor(x[e], dl, 64);
          const bool up = (i & k) == 0;
          const bool lower = (i & jj) == 0;
          x[e] = (lower == up) ? (x[e] < other ? x[e] : other) : (x[e] < other ? other : x[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) xch[tid * E + e] = x[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = tid * E + e;
          const uint64_t other = xch[i ^ jj];
          const bool up = (i & k) == 0;
          const bool lower = (i & jj) == 0;
          x[e] = (lower == up) ? (x[e] < other ? x[e] : other) : (x[e] < other ? other : x[e]);
        }
        __syncthreads();
      }
    }
  }
  // the previous key of each thread's first element (the last key of the thread before)
  uint64_t prev = __shfl_up(x[E - 1], 1, 64);
  if (lane == 63) wave_last[wid] = x[E - 1];
  __syncthreads();
  if (lane == 0) prev = wid > 0 ? wave_last[wid - 1] : ~0ull;
  int32_t* sp = spos + static_cast<int64_t>(b) * T;
  int32_t* si = sid + static_cast<int64_t>(b) * T;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = tid * E + e;
    const uint64_t pk = e > 0 ? x[e - 1] : prev;
    if (j < T) {
      sp[j] = static_cast<int32_t>(x[e] & 0xFFFFFFFFu);
      si[j] = static_cast<int32_t>(x[e] >> 32);
      cnt += (j == 0 || (pk >> 32) != (x[e] >> 32)) ? 1 : 0;
    }
  }
  // exclusive scan of cnt over the block
  int xs = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(xs, off, 64);
    if (lane >= off) xs += y;
  }
  if (lane == 63) red[wid] = xs;
  __syncthreads();
  int g = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kEmbSortThreads / 64; ++w) {
    g += w < wid ? red[w] : 0;
    total += red[w];
  }
  g += xs - cnt;
  int32_t* us = ustart + static_cast<int64_t>(b) * (T + 1);
  int32_t* ui = uid + static_cast<int64_t>(b) * T;
  int32_t* gp = gidp + static_cast<int64_t>(b) * T;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = tid * E + e;
    const uint64_t pk = e > 0 ? x[e - 1] : prev;
    if (j < T) {
      if (j == 0 || (pk >> 32) != (x[e] >> 32)) {
        us[g] = j;
        ui[g] = static_cast<int32_t>(x[e] >> 32);
        ++g;
      }
      gp[j] = g - 1;
    }
  }
  if (tid == 0) {
    ng[b] = total;
    us[total] = T;
  }
}

// Segmented sums of the delta rows in sorted order, one block per
// (2048-column chunk, split, sample); split s covers the sorted positions
// [s T / nsplit, (s + 1) T / nsplit), so a group may cross splits.  Within the
// block: a group wholly inside it is complete -- SUMS: its row sum goes to
// gsum[b][g]; otherwise its squared norm adds to part[b][s][chunk] (fp64).  The
// leading piece of a group that started before the split goes to head[b][s];
// the trailing piece of a group that goes on past the split (and is not the
// leading piece) goes to tail[b][s].  k_emb_combine joins the pieces.
template <typename TIn, bool VEC, bool SUMS>
__global__ void __launch_bounds__(kRmsThreads) k_emb_segments(
    const TIn* __restrict__ D, int T, int d, const int32_t* __restrict__ spos,
    const int32_t* __restrict__ sid, const int32_t* __restrict__ gidp, int nsplit,
    double* __restrict__ part, float* __restrict__ head, float* __restrict__ tail,
    float* __restrict__ gsum) {
  __shared__ double red[16];
  const int b = blockIdx.z, s = blockIdx.y, chunk = blockIdx.x, nchunk = gridDim.x;
  const int c0 = chunk * kRmsChunk + threadIdx.x * kRmsCols;
  const int cc = c0 < d ? c0 : 0;
  const int p_lo = static_cast<int>(static_cast<int64_t>(s) * T / nsplit);
  const int p_hi = static_cast<int>(static_cast<int64_t>(s + 1) * T / nsplit);
  const int32_t* sp = spos + static_cast<int64_t>(b) * T;
  const int32_t* si = sid + static_cast<int64_t>(b) * T;
  const TIn* db = D + static_cast<int64_t>(b) * T * d;
  const bool cont_before = p_lo > 0 && si[p_lo] == si[p_lo - 1];
  const bool cont_after = p_hi < T && si[p_hi] == si[p_hi - 1];
  int g = gidp[static_cast<int64_t>(b) * T + p_lo];  // group of the leading position
  float mask[kRmsCols];
#pragma unroll
  for (int k = 0; k < kRmsCols; ++k) mask[k] = (c0 + k < d) ? 1.f : 0.f;
  float run[kRmsCols];
#pragma unroll
  for (int k = 0; k < kRmsCols; ++k) run[k] = 0.f;
  double acc = 0.0;
  bool first = true;  // the open segment is the block's leading one
  float* hb = head + (static_cast<int64_t>(b) * nsplit + s) * d;
  float* tb = tail + (static_cast<int64_t>(b) * nsplit + s) * d;
  auto put = [&](float* dst) {
    if (c0 >= d) return;
    if (VEC) {
      *reinterpret_cast<float4*>(dst + c0) = make_float4(run[0], run[1], run[2], run[3]);
      *reinterpret_cast<float4*>(dst + c0 + 4) = make_float4(run[4], run[5], run[6], run[7]);
    } else {
#pragma unroll
      for (int k = 0; k < kRmsCols; ++k)
        if (c0 + k < d) dst[c0 + k] = run[k];
    }
  };
  // a segment ends inside the block: it is either the leading piece or complete
  auto close_inner = [&]() {
    if (first && cont_before) {
      put(hb);
    } else if (SUMS) {
      put(gsum + (static_cast<int64_t>(b) * T + g) * d);
    } else {
      float q = 0.f;
#pragma unroll
      for (int k = 0; k < kRmsCols; ++k) q = fmaf(mask[k] * run[k], run[k], q);
      acc += q;
    }
  };
  for (int p = p_lo; p < p_hi; p += 8) {
    int tt[8], idc[8], idp[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = p + u < p_hi ? p + u : p_hi - 1;
      tt[u] = sp[q];
      idc[u] = si[q];
      idp[u] = si[q > 0 ? q - 1 : 0];
    }
    float rows[8][kRmsCols];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const TIn* r = db + static_cast<int64_t>(tt[u]) * d;
      if (VEC) {
        load8(r + cc, rows[u]);
      } else {
#pragma unroll
        for (int k = 0; k < kRmsCols; ++k) rows[u][k] = load_f32(r + (cc + k < d ? cc + k : d - 1));
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (p + u < p_hi) {
        if (p + u > p_lo && idc[u] != idp[u]) {  // a group starts here
          close_inner();
          first = false;
          ++g;
#pragma unroll
          for (int k = 0; k < kRmsCols; ++k) run[k] = rows[u][k];
        } else {
#pragma unroll
          for (int k = 0; k < kRmsCols; ++k) run[k] += rows[u][k];
        }
      }
    }
  }
  // the last segment
  if (cont_after) {
    if (first && cont_before)
      put(hb);  // the whole split lies inside one group
    else
      put(tb);
  } else {
    close_inner();
  }
  if (!SUMS) {
    acc = block_sum_d(acc, red);
    if (threadIdx.x == 0) part[(static_cast<int64_t>(b) * nsplit + s) * nchunk + chunk] = acc;
  }
}

// Joins the pieces of the groups that cross splits, one thread per column,
// splits in order: a group's pieces are the trailing piece of the split where
// it starts, the leading pieces of the following splits, and it closes in the
// first of those with a group start inside or at the end of the last one.
// SUMS: the joined row sum goes to gsum[b][g]; otherwise its squared norm adds
// to cpart[b][chunk] (fp64).
constexpr int kEmbMaxSplits = 512;

template <bool SUMS>
__global__ void __launch_bounds__(256) k_emb_combine(
    const int32_t* __restrict__ gidp, int T, int d, int nsplit, const float* __restrict__ head,
    const float* __restrict__ tail, float* __restrict__ gsum, double* __restrict__ cpart) {
  __shared__ double red[16];
  // per split: bit 0 starts inside a group, bit 1 has a group start inside;
  // the group of its last position
  __shared__ int flags[kEmbMaxSplits];
  __shared__ int glast[kEmbMaxSplits];
  const int b = blockIdx.y, col = blockIdx.x * 256 + threadIdx.x;
  const int cc = col < d ? col : d - 1;
  const int32_t* gp = gidp + static_cast<int64_t>(b) * T;
  for (int s = threadIdx.x; s < nsplit; s += 256) {
    const int p0 = static_cast<int>(static_cast<int64_t>(s) * T / nsplit);
    const int p1 = static_cast<int>(static_cast<int64_t>(s + 1) * T / nsplit);
    const int g0 = gp[p0], g1 = gp[p1 - 1];
    const bool cb = p0 > 0 && gp[p0 - 1] == g0;
    flags[s] = (cb ? 1 : 0) | (g1 != g0 ? 2 : 0);
    glast[s] = g1;
  }
  __syncthreads();
  double acc = 0.0;
  float carry = 0.f;
  int gopen = -1;
  auto close = [&](int gg) {
    if (SUMS) {
      if (col < d) gsum[(static_cast<int64_t>(b) * T + gg) * d + col] = carry;
    } else {
      acc += col < d ? static_cast<double>(carry) * carry : 0.0;
    }
    carry = 0.f;
    gopen = -1;
  };
  // head and tail of eight splits in flight at a time (entries a split did
  // not write are loaded but not used; the split index is clamped)
  const float* hb = head + static_cast<int64_t>(b) * nsplit * d + cc;
  const float* tb = tail + static_cast<int64_t>(b) * nsplit * d + cc;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float hv[8], tv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sc = s0 + u < nsplit ? s0 + u : nsplit - 1;
      hv[u] = hb[static_cast<int64_t>(sc) * d];
      tv[u] = tb[static_cast<int64_t>(sc) * d];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u;
      if (s < nsplit) {
        const bool cb = flags[s] & 1, inner_start = flags[s] & 2;
        const bool ca = s + 1 < nsplit && (flags[s + 1] & 1);
        if (cb) {
          carry += hv[u];
          if (inner_start || !ca) close(gopen);
        }
        if (ca && (inner_start || !cb)) {
          carry = tv[u];
          gopen = glast[s];
        }
      }
    }
  }
  if (!SUMS) {
    acc = block_sum_d(acc, red);
    if (threadIdx.x == 0) cpart[static_cast<int64_t>(b) * gridDim.x + blockIdx.x] = acc;
  }
}

// n_sq[b] (= or +=) sum over splits and chunks of part[b][.][.] (fixed order).
__global__ void k_emb_final(const double* __restrict__ part, int nparts, float* __restrict__ n_sq,
                            int accumulate, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  double t = 0.0;
  for (int k = 0; k < nparts; ++k) t += part[static_cast<int64_t>(b) * nparts + k];
  n_sq[b] = static_cast<float>(accumulate ? static_cast<double>(n_sq[b]) + t : t);
}

hipError_t launch_emb_zero_norm(int B, float* n_sq, int accumulate, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_emb_final, dim3((B + 63) / 64), dim3(64), 0, s, nullptr, 0, n_sq,
                     accumulate, B);
  return hipGetLastError();
}

int emb_splits(int B, int T, int d) {
  const int chunks = (d + kRmsChunk - 1) / kRmsChunk;
  int want = (512 + B * chunks - 1) / (B * chunks > 0 ? B * chunks : 1);
  const int maxs = T / 32 > 0 ? T / 32 : 1;  // at least 32 positions per split
  if (want > maxs) want = maxs;
  if (want > kEmbMaxSplits) want = kEmbMaxSplits;
  return want < 1 ? 1 : want;
}

static int pow2_at_least(int T) {
  int p = 1;
  while (p < T) p <<= 1;
  return p;
}

hipError_t launch_emb_sort(const int32_t* ids, int B, int T, int32_t* spos, int32_t* sid,
                           int32_t* gidp, int32_t* ustart, int32_t* uid, int32_t* ng,
                           hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (T < 1 || T > kEmbMaxT) return hipErrorInvalidValue;
  const int N = pow2_at_least(T) > kEmbSortThreads ? pow2_at_least(T) : kEmbSortThreads;
#define DPRC_SORT(EE)                                                                             \
  hipLaunchKernelGGL(k_emb_sort<EE>, dim3(B), dim3(kEmbSortThreads), 0, s, ids, T, spos, sid,    \
                     gidp, ustart, uid, ng)
  switch (N / kEmbSortThreads) {
    case 1: DPRC_SORT(1); break;
    case 2: DPRC_SORT(2); break;
    case 4: DPRC_SORT(4); break;
    case 8: DPRC_SORT(8); break;
    default: DPRC_SORT(16); break;
  }
#undef DPRC_SORT
  return hipGetLastError();
}

int emb_combine_chunks(int d) { return (d + 255) / 256; }

// n_sq[b] (= or +=) sum of the fp64 partials part[b][.] and cpart[b][.] in order.
__global__ void k_emb_final2(const double* __restrict__ part, int nparts,
                             const double* __restrict__ cpart, int ncparts,
                             float* __restrict__ n_sq, int accumulate, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  double t = 0.0;
  for (int k = 0; k < nparts; ++k) t += part[static_cast<int64_t>(b) * nparts + k];
  for (int k = 0; k < ncparts; ++k) t += cpart[static_cast<int64_t>(b) * ncparts + k];
  n_sq[b] = static_cast<float>(accumulate ? static_cast<double>(n_sq[b]) + t : t);
}

template <typename TIn, bool SUMS>
static void emb_segments(const TIn* D, int B, int T, int d, const int32_t* spos,
                         const int32_t* sid, const int32_t* gidp, int nsplit, double* part,
                         float* head, float* tail, float* gsum, double* cpart, hipStream_t s) {
  const dim3 grid((d + kRmsChunk - 1) / kRmsChunk, nsplit, B);
  if (d % 8 == 0)
    hipLaunchKernelGGL((k_emb_segments<TIn, true, SUMS>), grid, dim3(kRmsThreads), 0, s, D, T, d,
                       spos, sid, gidp, nsplit, part, head, tail, gsum);
  else
    hipLaunchKernelGGL((k_emb_segments<TIn, false, SUMS>), grid, dim3(kRmsThreads), 0, s, D, T, d,
                       spos, sid, gidp, nsplit, part, head, tail, gsum);
  hipLaunchKernelGGL((k_emb_combine<SUMS>), dim3(emb_combine_chunks(d), B), dim3(256), 0, s, gidp,
                     T, d, nsplit, head, tail, gsum, cpart);
}

template <typename TIn>
hipError_t launch_emb_norm(const TIn* D, int B, int T, int d, const int32_t* spos,
                           const int32_t* sid, const int32_t* gidp, int nsplit, double* part,
                           float* head, float* tail, double* cpart, float* n_sq, int accumulate,
                           hipStream_t s) {
  if (B <= 0) return hipSuccess;
  emb_segments<TIn, false>(D, B, T, d, spos, sid, gidp, nsplit, part, head, tail, nullptr, cpart,
                           s);
  const int nchunk = (d + kRmsChunk - 1) / kRmsChunk;
  hipLaunchKernelGGL(k_emb_final2, dim3((B + 63) / 64), dim3(64), 0, s, part, nsplit * nchunk,
                     cpart, emb_combine_chunks(d), n_sq, accumulate, B);
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_emb_group_sums(const TIn* D, int B, int T, int d, const int32_t* spos,
                                 const int32_t* sid, const int32_t* gidp, int nsplit, float* head,
                                 float* tail, float* gsum, hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  emb_segments<TIn, true>(D, B, T, d, spos, sid, gidp, nsplit, nullptr, head, tail, gsum, nullptr,
                          s);
  return hipGetLastError();
}

// rowmap[b][v] = -1 for every v; then the group index of each id present in sample b.
__global__ void k_emb_rowmap_clear(int32_t* __restrict__ rowmap, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) rowmap[i] = -1;
}
__global__ void k_emb_rowmap_set(const int32_t* __restrict__ uid, const int32_t* __restrict__ ng,
                                 int T, int V, int32_t* __restrict__ rowmap) {
  const int b = blockIdx.y;
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= ng[b]) return;
  const int v = uid[static_cast<int64_t>(b) * T + g];
  if (v >= 0 && v < V) rowmap[static_cast<int64_t>(b) * V + v] = g;
}

// E[v][col] -= eta/B (S[v][col] + sigma C xi), S[v] = sum_b c_b gsum[b][group of v in b]
// (samples in order); xi from the noise stream of `layer`, flat index v d + col.
// VEC (d % 8 == 0): the row of E and the group sums move as float4, and E is
// loaded before the row-map lookups so that the two latencies overlap.
template <bool VEC>
__global__ void __launch_bounds__(kRmsThreads) k_emb_update(
    const float* __restrict__ gsum, int B, int T, int d, const int32_t* __restrict__ rowmap,
    int V, const float* __restrict__ cvec, float* __restrict__ E, float sigmaC, float eta_over_B,
    uint32_t k0, uint32_t k1, uint32_t layer) {
  __shared__ int grp[kRmsThreads];
  const int v = blockIdx.x;
  const int c0 = blockIdx.y * kRmsChunk + threadIdx.x * kRmsCols;
  const int cc = c0 < d ? c0 : 0;
  float* ev = E + static_cast<int64_t>(v) * d;
  float x[kRmsCols];
  if (VEC) {
    const float4 a = *reinterpret_cast<const float4*>(ev + cc);
    const float4 b4 = *reinterpret_cast<const float4*>(ev + cc + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b4.x; x[5] = b4.y; x[6] = b4.z; x[7] = b4.w;
  } else {
#pragma unroll
    for (int k = 0; k < kRmsCols; ++k) x[k] = ev[cc + k < d ? cc + k : d - 1];
  }
  float S[kRmsCols];
#pragma unroll
  for (int k = 0; k < kRmsCols; ++k) S[k] = 0.f;
  for (int i0 = 0; i0 < B; i0 += kRmsThreads) {
    const int i = i0 + threadIdx.x;
    grp[threadIdx.x] = i < B ? rowmap[static_cast<int64_t>(i) * V + v] : -1;
    __syncthreads();
    const int nb = B - i0 < kRmsThreads ? B - i0 : kRmsThreads;
    for (int j = 0; j < nb; ++j) {
      const int g = grp[j];
      if (g >= 0) {
        const int ib = i0 + j;
        const float* row = gsum + (static_cast<int64_t>(ib) * T + g) * d;
        const float cb = cvec[ib];
        float r[kRmsCols];
        if (VEC) {
          const float4 a = *reinterpret_cast<const float4*>(row + cc);
          const float4 b4 = *reinterpret_cast<const float4*>(row + cc + 4);
          r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
          r[4] = b4.x; r[5] = b4.y; r[6] = b4.z; r[7] = b4.w;
        } else {
#pragma unroll
          for (int k = 0; k < kRmsCols; ++k) r[k] = row[cc + k < d ? cc + k : d - 1];
        }
#pragma unroll
        for (int k = 0; k < kRmsCols; ++k) S[k] = fmaf(cb, r[k], S[k]);
      }
    }
    __syncthreads();
  }
  if (c0 >= d) return;
  const uint64_t e0 = static_cast<uint64_t>(v) * d + c0;
  if (VEC && (e0 & 3) == 0) {  // two whole counter groups
    float z[8];
    normals4(noise_counter(e0 >> 2, layer), k0, k1, z);
    normals4(noise_counter((e0 >> 2) + 1, layer), k0, k1, z + 4);
#pragma unroll
    for (int k = 0; k < kRmsCols; ++k) x[k] -= eta_over_B * fmaf(sigmaC, z[k], S[k]);
    *reinterpret_cast<float4*>(ev + c0) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(ev + c0 + 4) = make_float4(x[4], x[5], x[6], x[7]);
  } else {
    uint64_t gcur = ~0ull;
    float z[4];
#pragma unroll
    for (int k = 0; k < kRmsCols; ++k) {
      if (c0 + k < d) {
        const uint64_t e = e0 + k;
        if ((e >> 2) != gcur) {  // one Philox call per four consecutive elements
          gcur = e >> 2;
          normals4(noise_counter(gcur, layer), k0, k1, z);
        }
        ev[c0 + k] = x[k] - eta_over_B * fmaf(sigmaC, z[e & 3], S[k]);
      }
    }
  }
}

hipError_t launch_emb_update(const float* gsum, int B, int T, int d, const int32_t* uid,
                             const int32_t* ng, int32_t* rowmap, int V, const float* c, float* E,
                             float sigmaC, float eta_over_B, uint64_t seed, uint32_t layer,
                             hipStream_t s) {
  if (V <= 0) return hipSuccess;
  const int64_t nmap = static_cast<int64_t>(B) * V;
  if (B > 0 && T > 0) {
    hipLaunchKernelGGL(k_emb_rowmap_clear, dim3(static_cast<unsigned>((nmap + 255) / 256)),
                       dim3(256), 0, s, rowmap, nmap);
    hipLaunchKernelGGL(k_emb_rowmap_set, dim3((T + 255) / 256, B), dim3(256), 0, s, uid, ng, T, V,
                       rowmap);
  }
  const dim3 grid(V, (d + kRmsChunk - 1) / kRmsChunk);
  const int Bu = T > 0 ? B : 0;  // no tokens: no sample contributes
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  if (d % 8 == 0)
    hipLaunchKernelGGL(k_emb_update<true>, grid, dim3(kRmsThreads), 0, s, gsum, Bu, T, d, rowmap,
                       V, c, E, sigmaC, eta_over_B, k0, k1, layer);
  else
    hipLaunchKernelGGL(k_emb_update<false>, grid, dim3(kRmsThreads), 0, s, gsum, Bu, T, d, rowmap,
                       V, c, E, sigmaC, eta_over_B, k0, k1, layer);
  return hipGetLastError();
}

#define DPRC_EMB_INSTANTIATE(TIn)                                                                  \
  template hipError_t launch_emb_norm<TIn>(const TIn*, int, int, int, const int32_t*,            \
                                           const int32_t*, const int32_t*, int, double*, float*,  \
                                           float*, double*, float*, int, hipStream_t);            \
  template hipError_t launch_emb_group_sums<TIn>(const TIn*, int, int, int, const int32_t*,      \
                                                 const int32_t*, const int32_t*, int, float*,     \
                                                 float*, float*, hipStream_t);
DPRC_EMB_INSTANTIATE(float)
DPRC_EMB_INSTANTIATE(bf16_t)

}  // namespace dprc
