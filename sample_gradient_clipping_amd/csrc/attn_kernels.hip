// Forward pass and backward pass 1 of a Llama attention block on gfx950 (the
// randomized-clipping summary, section アルゴリズム的フロー, steps 1-2): rotary
// position embedding, and causal grouped-query attention with head width 64 as
// flash-style tiles (no T x T matrix in memory); T a multiple of 128.
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
// LDS tiles (64 x 64 bf16, 8 KB) are row-major with the 16-byte chunk c of row
// r stored at chunk position c ^ sw(r).  The LDS has 64 banks of 4 bytes, so a
// 256-byte bank line holds two tile rows.  Measured on gfx950: an 8-byte read
// (plain or ds_read_b64_tr_b16) is served 32 contiguous lanes per pass; a
// 16-byte read 16 lanes per pass, those of l ^ span{1, 2, 12, 20} (lane 0
// with lanes 1-3, 12-15, 20-23 and 24-27).  sw makes both kinds of operand read
// conflict-free: the 16-byte reads of 16 consecutive rows, and the transposing
// reads that give V^T, Q^T, dO^T and K^T from the same row-major tiles.
#include <cmath>
#include <type_traits>

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

// Swizzle of row r.  A 16-byte read pass takes rows {0-3, 12-15} (mod 16) at
// one chunk x and rows {4-11} at chunk x ^ 1 (or the other way round); with
// sw(r) = r & 6 the 8 rows of each parity land on 8 different chunk positions
// of their bank line.  A transposing read pass takes 8 consecutive rows (from a
// multiple of 8) at one 32-byte chunk pair, and the 4 rows of each parity land
// on 4 different pairs.
__device__ __forceinline__ int sw(int r) { return r & 6; }

// Element offset of the 16-byte chunk c (columns 8 c .. 8 c + 7) of row r.
__device__ __forceinline__ int rm_off(int r, int c) { return r * kBlk + ((c ^ sw(r)) << 3); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 at_lds_v4i16;

// 8 contraction slots for the operand "row n = column n0 + (l % 16) of the tile,
// slots = tile rows 32 t + 4 grp .. + 3, then 32 t + 16 + 4 grp .. + 3", read from
// a row-major swizzled tile with two transposing reads: in each group of 16
// lanes, lane 4 j + c addresses row (base + j), columns n0 + 4 c .. + 3, and
// receives slot j of column n0 + (l % 16).
__device__ __forceinline__ u32x4 rd_rm_tr8(const bf16_t* tile, int n0, int t, int grp, int lane16) {
  const int j = lane16 >> 2, c = lane16 & 3;
  const int col = n0 + 4 * c;
  const int r0 = 32 * t + 4 * grp + j, r1 = r0 + 16;
  const bf16_t* p0 = tile + r0 * kBlk + ((((col >> 3) ^ sw(r0)) << 3) | (col & 7));
  const bf16_t* p1 = tile + r1 * kBlk + ((((col >> 3) ^ sw(r1)) << 3) | (col & 7));
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_v4i16*)(p0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_v4i16*)(p1));
  const u32x2 aa = __builtin_bit_cast(u32x2, a), bb = __builtin_bit_cast(u32x2, b);
  return u32x4{aa.x, aa.y, bb.x, bb.y};
}

// 16-byte read of chunk c of row r of a swizzled tile.
__device__ __forceinline__ u32x4 rd16(const bf16_t* tile, int r, int c) {
  return *(at_lds_u32x4*)(tile + rm_off(r, c));
}

__device__ __forceinline__ uint32_t pk(float a, float b) { return pack_bf16x2(a, b); }

// 2^x with v_exp_f32 alone: the softmax only takes it of x <= 0, where a result
// below 2^-126 flushing to zero changes nothing the bf16 products can see.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) void at_lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((at_lds_void*)(p)));
}

// One 1 KB global -> LDS DMA instruction: lane i's 16 global bytes land at LDS
// m0 + 16 i.  m0 is saved and restored around it.  As inline asm the load is not
// an LDS write the compiler would drain before LDS reads: the kernel counts
// these loads itself (vmcnt) and orders the stages with s_barrier.
__device__ __forceinline__ void dma16(const bf16_t* gp, uint32_t lds) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(gp), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}

// One 256-byte global -> LDS DMA instruction: lane i's 4 global bytes land at
// LDS m0 + 4 i (counted and ordered like dma16).
__device__ __forceinline__ void dma4(const float* gp, uint32_t lds) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(gp), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}

// s_waitcnt with vmcnt = N (other counters unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup order.  Causal attention gives the workgroups of one launch very
// different amounts of work; dispatching the largest first keeps the last
// dispatched ones short, so the CUs run out of work nearly together.  Both map
// the flat workgroup index (x fastest) to (block, head, sample).
__device__ __forceinline__ void heavy_first_q(int nx, int ny, int nz, int& qb, int& h, int& b) {
  const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  h = id % ny;
  const int rest = id / ny;
  b = rest % nz;
  qb = nx - 1 - rest / nz;
}

__device__ __forceinline__ void heavy_first_kv(int nx, int ny, int nz, int& kbk, int& g, int& b) {
  const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  g = id % ny;
  const int rest = id / ny;
  b = rest % nz;
  kbk = rest / nz;
}

// Max and sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes that
// hold one query's scores) with the row-swapping permutes: permlane32_swap of a
// value with itself leaves {x[l], x[l ^ 32]} in the two results at every lane,
// permlane16_swap {x[l], x[l ^ 16]}.
__device__ __forceinline__ float max_lanes_xor48(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_lanes_xor48(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------------------
// Forward: one workgroup = 128 queries of one head, wave w owns queries
// 16 w .. + 15; 64-key tiles of K (row-major) and V (row-major, read with
// transposing reads) come into LDS by DMA three tiles ahead of the one in use.
// Online softmax in the log2 domain; each lane keeps its own share of a
// query's normaliser, summed over the query's four lanes after the loop.
// ---------------------------------------------------------------------------
constexpr int kFwdQ = 128;
constexpr int kFwdStages = 4;
constexpr int kTileElems = kBlk * kBlk;  // one 64 x 64 tile

__global__ void __launch_bounds__(512) k_attn_fwd(const bf16_t* __restrict__ q,
                                                  const bf16_t* __restrict__ k,
                                                  const bf16_t* __restrict__ v, int T, int H,
                                                  int KV, float scale_log2,
                                                  bf16_t* __restrict__ o,
                                                  float* __restrict__ lse) {
  // stage s: K tile at KV_s[s][0], V tile at KV_s[s][1]
  __shared__ __attribute__((aligned(16))) bf16_t KVs[kFwdStages][2][kTileElems];
  // Heaviest work first: the workgroups of the last query block (the most key
  // tiles) of every (sample, head) are dispatched first, the first block's last.
  int qb, h, b;
  heavy_first_q(gridDim.x, gridDim.y, gridDim.z, qb, h, b);
  const int gkv = h / (H / KV);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int li = lane & 15, lg = lane >> 4;
  const int64_t ldq = static_cast<int64_t>(H) * kDh, ldk = static_cast<int64_t>(KV) * kDh;
  const int tq = qb * kFwdQ + w * 16 + li;  // this lane's query
  const bf16_t* qrow = q + (static_cast<int64_t>(b) * T + tq) * ldq + h * kDh;
  const u32x4 qf0 = *reinterpret_cast<const u32x4*>(qrow + 8 * lg);
  const u32x4 qf1 = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * lg);
  // Use the query fragments here, before the first DMA: the compiler then waits
  // for them now, and not (with a count that the DMA loads would inflate) inside
  // the tile loop.
  asm volatile("" ::"v"(qf0), "v"(qf1));

  // DMA: wave w fills rows 8 w .. 8 w + 7 of the K tile and of the V tile, one
  // instruction each; lane i -> row 8 w + i / 8, LDS chunk i % 8, which holds
  // global chunk (i % 8) ^ sw(row).
  const int dr = 8 * w + (lane >> 3), dp = lane & 7;
  const int64_t kv0 = static_cast<int64_t>(b) * T * ldk + gkv * kDh + dr * ldk + 8 * (dp ^ sw(dr));
  const bf16_t* kg = k + kv0;
  const bf16_t* vg = v + kv0;
  const int nkt = (qb * kFwdQ + kFwdQ) / kBlk;  // key tiles up to the diagonal
  auto issue = [&](int kt) {
    const int64_t off = static_cast<int64_t>(kt) * kBlk * ldk;
    bf16_t* st = &KVs[kt % kFwdStages][0][0];
    dma16(kg + off, lds_addr(st + 8 * w * kBlk));
    dma16(vg + off, lds_addr(st + kTileElems + 8 * w * kBlk));
  };
  issue(0);
  if (nkt > 1) issue(1);
  if (nkt > 2) issue(2);

  float m = -INFINITY, l = 0.f;  // l: this lane's share of the normaliser
  f32x4 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int qlast = qb * kFwdQ + w * 16 + 15;  // the wave's last query

  // One key tile in LDS stage S (a constant, so that every LDS address below is
  // a per-lane register plus an immediate).
  auto tile = [&](int kt, auto stage) {
    constexpr int S = decltype(stage)::value;
    // this wave's loads of tile kt are done (those of kt + 1, kt + 2 may be in
    // flight); after the barrier every wave's are, and every wave is done with
    // the stage of tile kt - 1, which tile kt + 3 refills
    const int ahead = nkt - 1 - kt;
    if (ahead >= 2)
      wait_vm<4>();
    else if (ahead == 1)
      wait_vm<2>();
    else
      wait_vm<0>();
    bar();
    if (kt + 3 < nkt) issue(kt + 3);
    if (kt * kBlk > qlast) return;  // every key of the tile is after the wave's queries
    const bf16_t* Ks = &KVs[S][0][0];
    const bf16_t* Vs = Ks + kTileElems;

    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int r = kb * 16 + li;
      s[kb] = mma(rd16(Ks, r, lg), qf0, f32x4{0.f, 0.f, 0.f, 0.f});
      s[kb] = mma(rd16(Ks, r, 4 + lg), qf1, s[kb]);
    }
    // raw scores; the scale (> 0) goes into the max and the exponent's fma.  The
    // causal mask only on the tiles that reach past the wave's first query (a
    // wave-uniform branch).
    if ((kt + 1) * kBlk > qb * kFwdQ + w * 16) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt * kBlk + kb * 16 + 4 * lg + r > tq) s[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_lanes_xor48(mx);  // over the four lanes of this query
    const float mn = fmaxf(m, mx * scale_log2);
    const float alpha = ex2(m - mn);
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = ex2(fmaf(s[kb][r], scale_log2, -mn));
        s[kb][r] = p;
        sum += p;
      }
    l = l * alpha + sum;  // alpha is the same in the query's four lanes
    m = mn;
    if (__any(alpha != 1.0f)) {  // skipped when no lane's running max moved
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pb{pk(s[2 * t][0], s[2 * t][1]), pk(s[2 * t][2], s[2 * t][3]),
                     pk(s[2 * t + 1][0], s[2 * t + 1][1]), pk(s[2 * t + 1][2], s[2 * t + 1][3])};
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = mma(rd_rm_tr8(Vs, 16 * db, t, lg, li), pb, acc[db]);
    }
  };

  static_assert(kFwdStages == 4, "the loop below is unrolled over four stages");
  for (int kt = 0; kt < nkt; kt += 4) {
    tile(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nkt) tile(kt + 1, std::integral_constant<int, 1>{});
    if (kt + 2 < nkt) tile(kt + 2, std::integral_constant<int, 2>{});
    if (kt + 3 < nkt) tile(kt + 3, std::integral_constant<int, 3>{});
  }
  l = sum_lanes_xor48(l);

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
// registers: no atomics, a fixed order.  Each step's Q and dO tiles (swizzled
// row-major) and its 64 lse and D values come into LDS by DMA, one step ahead.
constexpr int kBkvLd = 4 * 64;  // floats per stage: per wave 16 lse, 16 D, 32 unused

__global__ void __launch_bounds__(256) k_attn_bwd_kv(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dvec,
    int T, int H, int KV, float scale_log2, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv) {
  // stage s: Q tile at QDs[s][0], dO tile at QDs[s][1], lse / D at LDs[s]
  __shared__ __attribute__((aligned(16))) bf16_t QDs[2][2][kTileElems];
  __shared__ __attribute__((aligned(16))) float LDs[2][kBkvLd];
  // Heaviest work first: the key blocks at the start of the sequence (the most
  // query blocks after them) of every (sample, head group) are dispatched first.
  int kbk, gkv, b;
  heavy_first_kv(gridDim.x, gridDim.y, gridDim.z, kbk, gkv, b);
  const int grp = H / KV;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int li = lane & 15, lg = lane >> 4;
  const int64_t ldq = static_cast<int64_t>(H) * kDh, ldk = static_cast<int64_t>(KV) * kDh;
  const int tk = kbk * kBlk + w * 16 + li;  // this lane's key
  const bf16_t* krow = k + (static_cast<int64_t>(b) * T + tk) * ldk + gkv * kDh;
  const bf16_t* vrow = v + (static_cast<int64_t>(b) * T + tk) * ldk + gkv * kDh;
  const u32x4 kf0 = *reinterpret_cast<const u32x4*>(krow + 8 * lg);
  const u32x4 kf1 = *reinterpret_cast<const u32x4*>(krow + 32 + 8 * lg);
  const u32x4 vf0 = *reinterpret_cast<const u32x4*>(vrow + 8 * lg);
  const u32x4 vf1 = *reinterpret_cast<const u32x4*>(vrow + 32 + 8 * lg);
  // Use the per-lane operands before the first DMA, so that the compiler waits
  // for them here and not, with counts the DMA loads would inflate, in the loop.
  asm volatile("" ::"v"(kf0), "v"(kf1), "v"(vf0), "v"(vf1));
  constexpr float kLog2e = 1.4426950408889634f;

  // DMA: wave w fills rows 16 w .. 16 w + 15 of the Q and dO tiles (two
  // instructions each, as in the dQ kernel) and, with one 4-byte-per-lane
  // instruction, the lse (lanes 0-15) and D (lanes 16-31) of queries
  // 16 w .. + 15; lanes 32-63 repeat lanes 0-31 into the unused half.
  // Lane i of instruction u -> row 16 w + 8 u + i / 8, LDS chunk i % 8, which
  // holds global chunk (i % 8) ^ sw(row) (sw(row + 8) = sw(row)).
  const int dr = 16 * w + (lane >> 3), dp = lane & 7;
  const int64_t qd0 = dr * ldq + 8 * (dp ^ sw(dr));
  const int l32 = lane & 31;
  const float* ldsrc = (l32 < 16 ? lse : Dvec) + 16 * w + (l32 & 15);
  const int nq = T / kBlk - kbk;  // query blocks from the diagonal on
  const int nit = grp * nq;
  auto issue = [&](int it) {
    const int j = it / nq;
    const int qb = kbk + (it - j * nq);
    const int h = gkv * grp + j;
    const int64_t off = (static_cast<int64_t>(b) * T + qb * kBlk) * ldq + h * kDh + qd0;
    const int st = it & 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      dma16(q + off + 8 * u * ldq, lds_addr(&QDs[st][0][(16 * w + 8 * u) * kBlk]));
      dma16(dO + off + 8 * u * ldq, lds_addr(&QDs[st][1][(16 * w + 8 * u) * kBlk]));
    }
    dma4(ldsrc + (static_cast<int64_t>(b) * H + h) * T + qb * kBlk, lds_addr(&LDs[st][64 * w]));
  };
  issue(0);

  f32x4 adk[4], adv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    adk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    adv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int kk = w * 16 + li;  // key within the block

  auto step = [&](int it, auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    // this wave's loads of step it are done; after the barrier every wave's
    // are, and every wave is done with the stage of step it - 1, which step
    // it + 1 refills
    wait_vm<0>();
    bar();
    if (it + 1 < nit) issue(it + 1);
    const bool diag = it % nq == 0;  // the query block of the workgroup's own keys
    const bf16_t* Qs = &QDs[S][0][0];
    const bf16_t* Ds = &QDs[S][1][0];
    f32x4 P[4], dS[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {  // 16-query blocks
      const int r0 = sb * 16 + li;
      f32x4 sc = mma(rd16(Qs, r0, lg), kf0, f32x4{0.f, 0.f, 0.f, 0.f});
      sc = mma(rd16(Qs, r0, 4 + lg), kf1, sc);
      f32x4 dpv = mma(rd16(Ds, r0, lg), vf0, f32x4{0.f, 0.f, 0.f, 0.f});
      dpv = mma(rd16(Ds, r0, 4 + lg), vf1, dpv);
      // lse and D of queries 16 sb + 4 lg .. + 3 (loaded by wave sb)
      const f32x4 L4 = *(const __attribute__((address_space(3))) f32x4*)(&LDs[S][64 * sb + 4 * lg]);
      const f32x4 D4 =
          *(const __attribute__((address_space(3))) f32x4*)(&LDs[S][64 * sb + 16 + 4 * lg]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = sb * 16 + 4 * lg + r;  // query within the block
        float p = ex2(fmaf(sc[r], scale_log2, -L4[r] * kLog2e));
        if (diag && kk > qq) p = 0.f;  // a select, no branch between the MFMAs
        P[sb][r] = p;
        dS[sb][r] = p * (dpv[r] - D4[r]);
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
        adv[db] = mma(rd_rm_tr8(Ds, 16 * db, t, lg, li), pb, adv[db]);
        adk[db] = mma(rd_rm_tr8(Qs, 16 * db, t, lg, li), sbv, adk[db]);
      }
    }
  };

  for (int it = 0; it < nit; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < nit) step(it + 1, std::integral_constant<int, 1>{});
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

// dQ of 128 queries of one head: wave w (of 8) owns queries 16 w .. + 15 (the
// query in the lane, S^T = K Q^T as in the forward); key tiles 0 .. the
// diagonal, K and V (both swizzled row-major) brought into LDS by DMA, double
// buffered; each tile serves the workgroup's 128 queries.
constexpr int kBqQ = 128;  // queries per workgroup

__global__ void __launch_bounds__(512) k_attn_bwd_q(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dvec,
    int T, int H, int KV, float scale_log2, bf16_t* __restrict__ dq) {
  // stage s: K tile at KVs[s][0], V tile at KVs[s][1]
  __shared__ __attribute__((aligned(16))) bf16_t KVs[2][2][kTileElems];
  // Heaviest work first: the workgroups of the last query block (the most key
  // tiles) of every (sample, head) are dispatched first, the first block's last.
  int qb, h, b;
  heavy_first_q(gridDim.x, gridDim.y, gridDim.z, qb, h, b);
  const int gkv = h / (H / KV);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int li = lane & 15, lg = lane >> 4;
  const int64_t ldq = static_cast<int64_t>(H) * kDh, ldk = static_cast<int64_t>(KV) * kDh;
  const int qfirst = qb * kBqQ + w * 16;  // the wave's first query
  const int tq = qfirst + li;
  const bf16_t* qrow = q + (static_cast<int64_t>(b) * T + tq) * ldq + h * kDh;
  const bf16_t* drow = dO + (static_cast<int64_t>(b) * T + tq) * ldq + h * kDh;
  const u32x4 qf0 = *reinterpret_cast<const u32x4*>(qrow + 8 * lg);
  const u32x4 qf1 = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * lg);
  const u32x4 df0 = *reinterpret_cast<const u32x4*>(drow + 8 * lg);
  const u32x4 df1 = *reinterpret_cast<const u32x4*>(drow + 32 + 8 * lg);
  const int64_t si = (static_cast<int64_t>(b) * H + h) * T + tq;
  const float lq = lse[si] * 1.4426950408889634f, dd = Dvec[si];
  // Use the per-lane operands before the first DMA, so that the compiler waits
  // for them here and not, with counts the DMA loads would inflate, in the loop.
  asm volatile("" ::"v"(qf0), "v"(qf1), "v"(df0), "v"(df1), "v"(lq), "v"(dd));

  // DMA: wave w fills rows 8 w .. 8 w + 7 of the K and V tiles, one instruction
  // each; lane i -> row 8 w + i / 8, LDS chunk i % 8, which holds global chunk
  // (i % 8) ^ sw(row).
  const int dr = 8 * w + (lane >> 3), dp = lane & 7;
  const int64_t kv0 = static_cast<int64_t>(b) * T * ldk + gkv * kDh + dr * ldk + 8 * (dp ^ sw(dr));
  const bf16_t* kg = k + kv0;
  const bf16_t* vg = v + kv0;
  const int nkt = (qb * kBqQ + kBqQ) / kBlk;  // key tiles up to the diagonal
  auto issue = [&](int kt) {
    const int64_t off = static_cast<int64_t>(kt) * kBlk * ldk;
    bf16_t* st = &KVs[kt & 1][0][0];
    dma16(kg + off, lds_addr(st + 8 * w * kBlk));
    dma16(vg + off, lds_addr(st + kTileElems + 8 * w * kBlk));
  };
  issue(0);

  f32x4 adq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) adq[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int qlast = qfirst + 15;

  auto tile = [&](int kt, auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    // this wave's loads of tile kt are done; after the barrier every wave's are,
    // and every wave is done with the stage of tile kt - 1, which tile kt + 1
    // refills
    wait_vm<0>();
    bar();
    if (kt + 1 < nkt) issue(kt + 1);
    if (kt * kBlk > qlast) return;  // every key of the tile is after the wave's queries
    const bool diag = (kt + 1) * kBlk > qfirst;  // some key after the wave's first query
    const bf16_t* Ks = &KVs[S][0][0];
    const bf16_t* Vs = Ks + kTileElems;
    f32x4 dS[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int r0 = kb * 16 + li;
      f32x4 st = mma(rd16(Ks, r0, lg), qf0, f32x4{0.f, 0.f, 0.f, 0.f});
      st = mma(rd16(Ks, r0, 4 + lg), qf1, st);
      f32x4 dpv = mma(rd16(Vs, r0, lg), df0, f32x4{0.f, 0.f, 0.f, 0.f});
      dpv = mma(rd16(Vs, r0, 4 + lg), df1, dpv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = ex2(fmaf(st[r], scale_log2, -lq));
        if (diag && kt * kBlk + kb * 16 + 4 * lg + r > tq) p = 0.f;  // a select, no branch
        dS[kb][r] = p * (dpv[r] - dd);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 sbv{pk(dS[2 * t][0], dS[2 * t][1]), pk(dS[2 * t][2], dS[2 * t][3]),
                      pk(dS[2 * t + 1][0], dS[2 * t + 1][1]), pk(dS[2 * t + 1][2], dS[2 * t + 1][3])};
#pragma unroll
      for (int db = 0; db < 4; ++db) adq[db] = mma(rd_rm_tr8(Ks, 16 * db, t, lg, li), sbv, adq[db]);
    }
  };

  for (int kt = 0; kt < nkt; kt += 2) {  // nkt is even
    tile(kt, std::integral_constant<int, 0>{});
    tile(kt + 1, std::integral_constant<int, 1>{});
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
// cosine are taken in fp64.  A block takes 8 rows: first one thread per (row,
// pair) forms the row's 32 cosines and sines (shared by all heads) in LDS, then
// one thread per (row, head, 8 pairs) rotates.
// ---------------------------------------------------------------------------
constexpr int kRopeRows = 8;  // rows per block step; 8 x 32 angles = one per thread

__global__ void __launch_bounds__(256) k_rope(bf16_t* __restrict__ x, int64_t M, int T, int nh,
                                              double log_base, int inverse) {
  __shared__ float cs_l[kRopeRows][32], sn_l[kRopeRows][32];
  const int64_t ngroups = (M + kRopeRows - 1) / kRopeRows;
  const int items = kRopeRows * nh * 4;
  for (int64_t rg = blockIdx.x; rg < ngroups; rg += gridDim.x) {
    const int64_t row0 = rg * kRopeRows;
    {
      const int r = threadIdx.x >> 5, i = threadIdx.x & 31;
      const int64_t row = row0 + r;
      if (row < M) {
        const double pos = static_cast<double>(row % T);
        const double ang = pos * exp(-static_cast<double>(i) / 32.0 * log_base);
        double sd, cd;
        sincos(ang, &sd, &cd);
        cs_l[r][i] = static_cast<float>(cd);
        sn_l[r][i] = static_cast<float>(inverse ? -sd : sd);
      }
    }
    __syncthreads();
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
      const int r = it / (nh * 4);
      const int rem = it - r * nh * 4;
      const int64_t row = row0 + r;
      if (row >= M) continue;
      const int hd = rem >> 2, i0 = (rem & 3) * 8;
      bf16_t* p = x + row * nh * kDh + hd * kDh;
      const u32x4 a = *reinterpret_cast<const u32x4*>(p + i0);
      const u32x4 c = *reinterpret_cast<const u32x4*>(p + 32 + i0);
      float x1[8], x2[8], y1[8], y2[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        x1[2 * e2] = __uint_as_float(a[e2] << 16);
        x1[2 * e2 + 1] = __uint_as_float(a[e2] & 0xFFFF0000u);
        x2[2 * e2] = __uint_as_float(c[e2] << 16);
        x2[2 * e2 + 1] = __uint_as_float(c[e2] & 0xFFFF0000u);
      }
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const float cs = cs_l[r][i0 + e2], sn = sn_l[r][i0 + e2];
        y1[e2] = x1[e2] * cs - x2[e2] * sn;
        y2[e2] = x2[e2] * cs + x1[e2] * sn;
      }
      *reinterpret_cast<u32x4*>(p + i0) =
          u32x4{pk(y1[0], y1[1]), pk(y1[2], y1[3]), pk(y1[4], y1[5]), pk(y1[6], y1[7])};
      *reinterpret_cast<u32x4*>(p + 32 + i0) =
          u32x4{pk(y2[0], y2[1]), pk(y2[2], y2[3]), pk(y2[4], y2[5]), pk(y2[6], y2[7])};
    }
    __syncthreads();  // the angles of this step are read before the next step writes
  }
}

}  // namespace

bool attn_shape_ok(int T, int H, int KV) {
  return T > 0 && T % kFwdQ == 0 && H > 0 && KV > 0 && H % KV == 0 && T <= (1 << 20);
}

hipError_t launch_rope(bf16_t* x, int64_t M, int T, int nh, double base, bool inverse,
                       hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (T <= 0 || nh <= 0 || !(base > 1.0)) return hipErrorInvalidValue;
  const int64_t groups = (M + kRopeRows - 1) / kRopeRows;
  const int64_t blocks = groups < 8192 ? groups : 8192;
  hipLaunchKernelGGL(k_rope, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x, M, T, nh,
                     std::log(base), inverse ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const bf16_t* q, const bf16_t* k, const bf16_t* v, int B, int T, int H,
                           int KV, bf16_t* o, float* lse, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!attn_shape_ok(T, H, KV)) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
  hipLaunchKernelGGL(k_attn_fwd, dim3(T / kFwdQ, H, B), dim3(512), 0, s, q, k, v, T, H, KV,
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
  hipLaunchKernelGGL(k_attn_bwd_q, dim3(T / kBqQ, H, B), dim3(512), 0, s, q, k, v, dO, lse, Dvec,
                     T, H, KV, scale_log2, dq);
  return hipGetLastError();
}

}  // namespace dprc
