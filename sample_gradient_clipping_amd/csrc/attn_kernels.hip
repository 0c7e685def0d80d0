// Forward pass and backward pass 1 of a Llama attention block on gfx950 (the
// randomized-clipping summary, section アルゴリズム的フロー, steps 1-2): rotary
// position embedding, and causal grouped-query attention with head width 64 as
// flash-style tiles (no T x T matrix in memory).
//
// MFMA facts used (v_mfma_f32_16x16x32_bf16, wave64): lane l supplies row
// l % 16 of the first operand and column l % 16 of the second, each with the 8
// contraction slots 8 (l / 16) .. + 7; lane l receives D[4 (l / 16) + r][l % 16]
// in accumulator register r.  Which contraction index sits in which slot is free
// as long as both operands agree.
//
// Layout trick.  Scores are computed transposed, S^T = K Q^T, so a lane holds
// the scores of ONE query (column l % 16) for the 16 keys 16 kb + 4 (l / 16) + r
// (kb = 0..3, r = 0..3): the softmax statistics of a query live in the four
// lanes l % 16 and need two cross-lane shuffles.  For a 32-key step t those
// lanes already hold the keys 32 t + 4 (l / 16) + r and 32 t + 16 + 4 (l / 16) + r:
// exactly 8 contraction slots, so the probabilities are the second operand of
// O^T += V^T P^T straight from registers, and V^T's rows come from LDS with the
// same key order.  Every product of the backward pass uses one of these two
// orientations (query in the lane, or key in the lane) the same way.
//
// LDS tiles (64 x 64 bf16, 8 KB): row-major with the 16-byte chunk c of row r
// at c ^ (r & 7) (16-byte reads of 8 consecutive rows hit distinct banks), or
// transposed (line = column) with the 8-byte chunk c of line n at c ^ (n & 15)
// (8-byte reads of 16 consecutive lines hit distinct banks).
#include <cmath>

#include "common.h"
#include "internal.h"

namespace dprc {
namespace {

constexpr int kDh = 64;   // head width
constexpr int kBlk = 64;  // queries per workgroup, keys per tile

typedef __attribute__((address_space(3))) const u32x4 at_lds_u32x4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2 at_lds_u32x2;
typedef __attribute__((address_space(3))) u32x4 at_lds_u32x4_w;

__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Element offset of the 16-byte chunk c (columns 8 c .. 8 c + 7) of row r in a
// row-major swizzled tile.
__device__ __forceinline__ int rm_off(int r, int c) { return r * kBlk + ((c ^ (r & 7)) << 3); }
// Element offset of (row, column) in a transposed swizzled tile.
__device__ __forceinline__ int tr_off(int row, int col) {
  return col * kBlk + ((((row >> 2) ^ (col & 15))) << 2) + (row & 3);
}

__device__ __forceinline__ u32x4 rd16(const bf16_t* tile, int r, int c) {
  return *(at_lds_u32x4*)(tile + rm_off(r, c));
}
// 8 contraction slots of transposed line n: rows 32 t + 4 grp .. + 3, then
// 32 t + 16 + 4 grp .. + 3.
__device__ __forceinline__ u32x4 rd_tr8(const bf16_t* tile, int n, int t, int grp) {
  const u32x2 lo = *(at_lds_u32x2*)(tile + tr_off(32 * t + 4 * grp, n));
  const u32x2 hi = *(at_lds_u32x2*)(tile + tr_off(32 * t + 16 + 4 * grp, n));
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// 64 rows x 64 columns (row stride ld elements) from global into a row-major
// swizzled tile and/or a transposed one; 256 threads, two 16-byte chunks each.
template <bool RM, bool TR>
__device__ __forceinline__ void stage(const bf16_t* src, int64_t ld, bf16_t* rm, bf16_t* tr) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int id = threadIdx.x + 256 * j;
    const int r = id >> 3, c = id & 7;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + r * ld + 8 * c);
    if (RM) *(at_lds_u32x4_w*)(rm + rm_off(r, c)) = v;
    if (TR) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = v[e >> 1];
        tr[tr_off(r, 8 * c + e)] = static_cast<bf16_t>((e & 1) ? (w >> 16) : (w & 0xFFFFu));
      }
    }
  }
}

__device__ __forceinline__ uint32_t pk(float a, float b) { return pack_bf16x2(a, b); }

// ---------------------------------------------------------------------------
// Forward: one workgroup = 64 queries of one head; wave w owns queries
// 16 w .. + 15.  Online softmax in the log2 domain.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_attn_fwd(const bf16_t* __restrict__ q,
                                                  const bf16_t* __restrict__ k,
                                                  const bf16_t* __restrict__ v, int T, int H,
                                                  int KV, float scale_log2,
                                                  bf16_t* __restrict__ o,
                                                  float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kBlk * kBlk];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[kBlk * kBlk];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int gkv = h / (H / KV);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t ldq = static_cast<int64_t>(H) * kDh, ldk = static_cast<int64_t>(KV) * kDh;
  const int tq = qb * kBlk + w * 16 + li;  // this lane's query
  const bf16_t* qrow = q + (static_cast<int64_t>(b) * T + tq) * ldq + h * kDh;
  const u32x4 qf0 = *reinterpret_cast<const u32x4*>(qrow + 8 * lg);
  const u32x4 qf1 = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * lg);

  float m = -INFINITY, l = 0.f;
  f32x4 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt <= qb; ++kt) {
    __syncthreads();
    const int64_t krow0 = static_cast<int64_t>(b) * T + kt * kBlk;
    stage<true, false>(k + krow0 * ldk + gkv * kDh, ldk, Ks, nullptr);
    stage<false, true>(v + krow0 * ldk + gkv * kDh, ldk, nullptr, Vt);
    __syncthreads();

    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int r = kb * 16 + li;
      s[kb] = mma(rd16(Ks, r, lg), qf0, f32x4{0.f, 0.f, 0.f, 0.f});
      s[kb] = mma(rd16(Ks, r, 4 + lg), qf1, s[kb]);
    }
    float mx = -INFINITY;
    const int qq = w * 16 + li;  // query within the block
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[kb][r] * scale_log2;
        if (kt == qb && kb * 16 + 4 * lg + r > qq) x = -INFINITY;
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[kb][r] - mn);
        s[kb][r] = p;
        sum += p;
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    l = l * alpha + sum;
    m = mn;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] *= alpha;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pb{pk(s[2 * t][0], s[2 * t][1]), pk(s[2 * t][2], s[2 * t][3]),
                     pk(s[2 * t + 1][0], s[2 * t + 1][1]), pk(s[2 * t + 1][2], s[2 * t + 1][3])};
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = mma(rd_tr8(Vt, 16 * db + li, t, lg), pb, acc[db]);
    }
  }

  const float inv = 1.0f / l;
  bf16_t* orow = o + (static_cast<int64_t>(b) * T + tq) * ldq + h * kDh;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const f32x4 a = acc[db] * inv;
    *reinterpret_cast<uint2*>(orow + 16 * db + 4 * lg) = uint2{pk(a[0], a[1]), pk(a[2], a[3])};
  }
  if (lg == 0)
    lse[(static_cast<int64_t>(b) * H + h) * T + tq] = (m + log2f(l)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// Backward.  Dvec[b][h][t] = sum over the head's 64 columns of dO * O.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_attn_bwd_dot(const bf16_t* __restrict__ dO,
                                                      const bf16_t* __restrict__ O, int64_t M,
                                                      int T, int H, float* __restrict__ Dvec) {
  const int64_t n = M * H;
  for (int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; id < n;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = id / H;
    const int h = static_cast<int>(id - row * H);
    const bf16_t* a = dO + row * H * kDh + h * kDh;
    const bf16_t* c = O + row * H * kDh + h * kDh;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(a + 8 * j);
      const u32x4 y = *reinterpret_cast<const u32x4*>(c + 8 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += __uint_as_float(x[e] << 16) * __uint_as_float(y[e] << 16);
        acc += __uint_as_float(x[e] & 0xFFFF0000u) * __uint_as_float(y[e] & 0xFFFF0000u);
      }
    }
    const int64_t b = row / T, t = row - b * T;
    Dvec[(b * H + h) * T + t] = acc;
  }
}

// dK, dV of 64 keys of one key/value head: wave w owns keys 16 w .. + 15 (the
// key in the lane, S = Q K^T), and the workgroup walks the group's query heads
// and, causally, the query blocks from its own on.  The head sums stay in
// registers: no atomics, a fixed order.
__global__ void __launch_bounds__(256) k_attn_bwd_kv(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dvec,
    int T, int H, int KV, float scale_log2, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv) {
  __shared__ __attribute__((aligned(16))) bf16_t Qs[kBlk * kBlk];
  __shared__ __attribute__((aligned(16))) bf16_t Qt[kBlk * kBlk];
  __shared__ __attribute__((aligned(16))) bf16_t Ds[kBlk * kBlk];
  __shared__ __attribute__((aligned(16))) bf16_t Dt[kBlk * kBlk];
  __shared__ float Ls[kBlk], Dd[kBlk];
  const int kbk = blockIdx.x, gkv = blockIdx.y, b = blockIdx.z;
  const int grp = H / KV;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t ldq = static_cast<int64_t>(H) * kDh, ldk = static_cast<int64_t>(KV) * kDh;
  const int tk = kbk * kBlk + w * 16 + li;  // this lane's key
  const bf16_t* krow = k + (static_cast<int64_t>(b) * T + tk) * ldk + gkv * kDh;
  const bf16_t* vrow = v + (static_cast<int64_t>(b) * T + tk) * ldk + gkv * kDh;
  const u32x4 kf0 = *reinterpret_cast<const u32x4*>(krow + 8 * lg);
  const u32x4 kf1 = *reinterpret_cast<const u32x4*>(krow + 32 + 8 * lg);
  const u32x4 vf0 = *reinterpret_cast<const u32x4*>(vrow + 8 * lg);
  const u32x4 vf1 = *reinterpret_cast<const u32x4*>(vrow + 32 + 8 * lg);
  constexpr float kLog2e = 1.4426950408889634f;

  f32x4 adk[4], adv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    adk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    adv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int kk = w * 16 + li;  // key within the block
  for (int j = 0; j < grp; ++j) {
    const int h = gkv * grp + j;
    for (int qb = kbk; qb < T / kBlk; ++qb) {
      __syncthreads();
      const int64_t qrow0 = static_cast<int64_t>(b) * T + qb * kBlk;
      stage<true, true>(q + qrow0 * ldq + h * kDh, ldq, Qs, Qt);
      stage<true, true>(dO + qrow0 * ldq + h * kDh, ldq, Ds, Dt);
      if (threadIdx.x < kBlk) {
        const int64_t si = (static_cast<int64_t>(b) * H + h) * T + qb * kBlk + threadIdx.x;
        Ls[threadIdx.x] = lse[si] * kLog2e;
        Dd[threadIdx.x] = Dvec[si];
      }
      __syncthreads();
      f32x4 P[4], dS[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {  // 16-query blocks
        const int r0 = sb * 16 + li;
        f32x4 sc = mma(rd16(Qs, r0, lg), kf0, f32x4{0.f, 0.f, 0.f, 0.f});
        sc = mma(rd16(Qs, r0, 4 + lg), kf1, sc);
        f32x4 dp = mma(rd16(Ds, r0, lg), vf0, f32x4{0.f, 0.f, 0.f, 0.f});
        dp = mma(rd16(Ds, r0, 4 + lg), vf1, dp);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qq = sb * 16 + 4 * lg + r;  // query within the block
          float p = exp2f(sc[r] * scale_log2 - Ls[qq]);
          if (qb == kbk && kk > qq) p = 0.f;
          P[sb][r] = p;
          dS[sb][r] = p * (dp[r] - Dd[qq]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 pb{pk(P[2 * t][0], P[2 * t][1]), pk(P[2 * t][2], P[2 * t][3]),
                       pk(P[2 * t + 1][0], P[2 * t + 1][1]), pk(P[2 * t + 1][2], P[2 * t + 1][3])};
        const u32x4 sbv{pk(dS[2 * t][0], dS[2 * t][1]), pk(dS[2 * t][2], dS[2 * t][3]),
                        pk(dS[2 * t + 1][0], dS[2 * t + 1][1]),
                        pk(dS[2 * t + 1][2], dS[2 * t + 1][3])};
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          adv[db] = mma(rd_tr8(Dt, 16 * db + li, t, lg), pb, adv[db]);
          adk[db] = mma(rd_tr8(Qt, 16 * db + li, t, lg), sbv, adk[db]);
        }
      }
    }
  }
  bf16_t* dkrow = dk + (static_cast<int64_t>(b) * T + tk) * ldk + gkv * kDh;
  bf16_t* dvrow = dv + (static_cast<int64_t>(b) * T + tk) * ldk + gkv * kDh;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const f32x4 a = adk[db] * 0.125f;  // 1 / sqrt(64)
    *reinterpret_cast<uint2*>(dkrow + 16 * db + 4 * lg) = uint2{pk(a[0], a[1]), pk(a[2], a[3])};
    const f32x4 c = adv[db];
    *reinterpret_cast<uint2*>(dvrow + 16 * db + 4 * lg) = uint2{pk(c[0], c[1]), pk(c[2], c[3])};
  }
}

// dQ of 64 queries of one head: wave w owns queries 16 w .. + 15 (the query in
// the lane, S^T = K Q^T as in the forward); key tiles 0 .. the diagonal.
__global__ void __launch_bounds__(256) k_attn_bwd_q(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dvec,
    int T, int H, int KV, float scale_log2, bf16_t* __restrict__ dq) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kBlk * kBlk];
  __shared__ __attribute__((aligned(16))) bf16_t Kt[kBlk * kBlk];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[kBlk * kBlk];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int gkv = h / (H / KV);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t ldq = static_cast<int64_t>(H) * kDh, ldk = static_cast<int64_t>(KV) * kDh;
  const int tq = qb * kBlk + w * 16 + li;
  const bf16_t* qrow = q + (static_cast<int64_t>(b) * T + tq) * ldq + h * kDh;
  const bf16_t* drow = dO + (static_cast<int64_t>(b) * T + tq) * ldq + h * kDh;
  const u32x4 qf0 = *reinterpret_cast<const u32x4*>(qrow + 8 * lg);
  const u32x4 qf1 = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * lg);
  const u32x4 df0 = *reinterpret_cast<const u32x4*>(drow + 8 * lg);
  const u32x4 df1 = *reinterpret_cast<const u32x4*>(drow + 32 + 8 * lg);
  const int64_t si = (static_cast<int64_t>(b) * H + h) * T + tq;
  const float lq = lse[si] * 1.4426950408889634f, dd = Dvec[si];

  f32x4 adq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) adq[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int qq = w * 16 + li;
  for (int kt = 0; kt <= qb; ++kt) {
    __syncthreads();
    const int64_t krow0 = static_cast<int64_t>(b) * T + kt * kBlk;
    stage<true, true>(k + krow0 * ldk + gkv * kDh, ldk, Ks, Kt);
    stage<true, false>(v + krow0 * ldk + gkv * kDh, ldk, Vs, nullptr);
    __syncthreads();
    f32x4 dS[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int r0 = kb * 16 + li;
      f32x4 st = mma(rd16(Ks, r0, lg), qf0, f32x4{0.f, 0.f, 0.f, 0.f});
      st = mma(rd16(Ks, r0, 4 + lg), qf1, st);
      f32x4 dp = mma(rd16(Vs, r0, lg), df0, f32x4{0.f, 0.f, 0.f, 0.f});
      dp = mma(rd16(Vs, r0, 4 + lg), df1, dp);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = exp2f(st[r] * scale_log2 - lq);
        if (kt == qb && kb * 16 + 4 * lg + r > qq) p = 0.f;
        dS[kb][r] = p * (dp[r] - dd);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 sbv{pk(dS[2 * t][0], dS[2 * t][1]), pk(dS[2 * t][2], dS[2 * t][3]),
                      pk(dS[2 * t + 1][0], dS[2 * t + 1][1]), pk(dS[2 * t + 1][2], dS[2 * t + 1][3])};
#pragma unroll
      for (int db = 0; db < 4; ++db) adq[db] = mma(rd_tr8(Kt, 16 * db + li, t, lg), sbv, adq[db]);
    }
  }
  bf16_t* dqrow = dq + (static_cast<int64_t>(b) * T + tq) * ldq + h * kDh;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const f32x4 a = adq[db] * 0.125f;
    *reinterpret_cast<uint2*>(dqrow + 16 * db + 4 * lg) = uint2{pk(a[0], a[1]), pk(a[2], a[3])};
  }
}

// ---------------------------------------------------------------------------
// RoPE in place on x [B T][nh * 64]: in each head the pair (i, i + 32) is
// rotated by pos * base^(-i / 32), pos = row % T; the angle and its sine and
// cosine are taken in fp64.  One thread per (row, head, 8 pairs).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_rope(bf16_t* __restrict__ x, int64_t M, int T, int nh,
                                              double log_base, int inverse) {
  const int64_t n = M * nh * 4;
  for (int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; id < n;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = id / (nh * 4);
    const int rem = static_cast<int>(id - row * nh * 4);
    const int hd = rem >> 2, i0 = (rem & 3) * 8;
    const double pos = static_cast<double>(row % T);
    bf16_t* p = x + row * nh * kDh + hd * kDh;
    const u32x4 a = *reinterpret_cast<const u32x4*>(p + i0);
    const u32x4 c = *reinterpret_cast<const u32x4*>(p + 32 + i0);
    float x1[8], x2[8], y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x1[2 * e] = __uint_as_float(a[e] << 16);
      x1[2 * e + 1] = __uint_as_float(a[e] & 0xFFFF0000u);
      x2[2 * e] = __uint_as_float(c[e] << 16);
      x2[2 * e + 1] = __uint_as_float(c[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double ang = pos * exp(-static_cast<double>(i0 + e) / 32.0 * log_base);
      double sd, cd;
      sincos(ang, &sd, &cd);
      const float cs = static_cast<float>(cd), sn = static_cast<float>(inverse ? -sd : sd);
      y1[e] = x1[e] * cs - x2[e] * sn;
      y2[e] = x2[e] * cs + x1[e] * sn;
    }
    *reinterpret_cast<u32x4*>(p + i0) =
        u32x4{pk(y1[0], y1[1]), pk(y1[2], y1[3]), pk(y1[4], y1[5]), pk(y1[6], y1[7])};
    *reinterpret_cast<u32x4*>(p + 32 + i0) =
        u32x4{pk(y2[0], y2[1]), pk(y2[2], y2[3]), pk(y2[4], y2[5]), pk(y2[6], y2[7])};
  }
}

}  // namespace

bool attn_shape_ok(int T, int H, int KV) {
  return T > 0 && T % kBlk == 0 && H > 0 && KV > 0 && H % KV == 0 && T <= (1 << 20);
}

hipError_t launch_rope(bf16_t* x, int64_t M, int T, int nh, double base, bool inverse,
                       hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (T <= 0 || nh <= 0 || !(base > 1.0)) return hipErrorInvalidValue;
  const int64_t n = M * nh * 4;
  const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
  hipLaunchKernelGGL(k_rope, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x, M, T, nh,
                     std::log(base), inverse ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const bf16_t* q, const bf16_t* k, const bf16_t* v, int B, int T, int H,
                           int KV, bf16_t* o, float* lse, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!attn_shape_ok(T, H, KV)) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
  hipLaunchKernelGGL(k_attn_fwd, dim3(T / kBlk, H, B), dim3(256), 0, s, q, k, v, T, H, KV,
                     scale_log2, o, lse);
  return hipGetLastError();
}

size_t attn_bwd_scratch_bytes(int B, int T, int H) {
  return static_cast<size_t>(B) * H * T * sizeof(float);
}

hipError_t launch_attn_bwd(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* o,
                           const float* lse, const bf16_t* dO, int B, int T, int H, int KV,
                           float* Dvec, bf16_t* dq, bf16_t* dk, bf16_t* dv, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!attn_shape_ok(T, H, KV)) return hipErrorInvalidValue;
  const int64_t M = static_cast<int64_t>(B) * T;
  const int64_t n = M * H;
  const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
  hipLaunchKernelGGL(k_attn_bwd_dot, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, dO, o,
                     M, T, H, Dvec);
  const float scale_log2 = 1.4426950408889634f / 8.0f;
  hipLaunchKernelGGL(k_attn_bwd_kv, dim3(T / kBlk, KV, B), dim3(256), 0, s, q, k, v, dO, lse,
                     Dvec, T, H, KV, scale_log2, dk, dv);
  hipLaunchKernelGGL(k_attn_bwd_q, dim3(T / kBlk, H, B), dim3(256), 0, s, q, k, v, dO, lse, Dvec,
                     T, H, KV, scale_log2, dq);
  return hipGetLastError();
}

}  // namespace dprc
