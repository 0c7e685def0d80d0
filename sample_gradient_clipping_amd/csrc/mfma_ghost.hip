// Ghost-clipping baseline on MFMA (bf16 in, fp32 accumulate), gfx950.
//
//   n_i = sum_{s,t} (A_i A_i^T)_{st} (G_i G_i^T)_{st}
//
// (randomized-clipping summary, sections 問題定義 and 1. 複雑性の削減: ghost
// clipping works with T x T Gram products, O(T^2 (p + d)) work per sample; the
// trace identity of section 中核メカニズム makes it equal to ||A_i^T G_i||_F^2.)
//
// One workgroup per (sample, 256-token block S, 128-token block t) with
// t >= 2 S, which covers every token pair s <= t once.  It forms the 256 x 128
// tile of A A^T over the d features and then, in the same pipeline, the tile
// of G G^T over the p features; both stay in registers (8 waves of 64 x 64),
// and their elementwise product is summed with weight 2 for s < t, 1 for
// s = t and 0 for s > t (the Grams are symmetric).  Both Gram operands are
// token rows with the features contiguous, the MFMA operand layout as stored:
// 64-feature slabs of the 384 rows (one 128-byte cache line per row) come into
// LDS by DMA in three slots, one barrier per slab, and are read with 16-byte
// reads one k-step ahead of the products.  Rows past T (T % 256 = 128) are read
// from row T - 1 and weighted 0.
//
// Order: super-tiles of 4 S blocks x 8 t blocks (1024 x 1024 tokens, 32
// workgroups) are dealt to the eight XCDs one per XCD per round, so that the 32
// workgroups an XCD runs at a time share 2048 token rows in its L2 and the
// eight XCDs work on neighbouring super-tiles.
#include "common.h"
#include "internal.h"

namespace dprc {
namespace {

constexpr int kGs = 256;                      // tokens per S block (tile rows)
constexpr int kGt = 128;                      // tokens per t block (tile columns)
constexpr int kGk = 64;                       // features per slab
constexpr int kGRow = kGk * 2;                // 128 bytes of a row per slab
constexpr int kGStage = (kGs + kGt) * kGRow;  // 48 KB
constexpr int kGStages = 3;
constexpr int kSupS = 4, kSupT = 8;       // super-tile, in blocks
constexpr int kXcd = 8;

__shared__ __attribute__((aligned(16))) unsigned char g_lds[kGStages * kGStage];

typedef __attribute__((address_space(3))) void g_lds_void;
typedef __attribute__((address_space(3))) const u32x4 g_lds_u32x4;

__device__ __forceinline__ uint32_t g_lds_addr(const unsigned char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((g_lds_void*)(p)));
}

// Chunk c (16 bytes) of LDS row r sits at chunk position c ^ g_swz(r).  Two
// 128-byte rows share a 256-byte bank line; a 16-byte read pass takes rows
// {0-3, 12-15} (mod 16) at one chunk and rows {4-11} at the neighbouring chunk,
// and with this swizzle the 8 rows of each parity land on 8 different chunk
// positions.
__device__ __forceinline__ int g_swz(int r) { return r & 6; }

template <int N>
__device__ __forceinline__ void g_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most 6 k of this wave's DMA loads (k slabs) are in flight.
__device__ __forceinline__ void g_wait_slabs(int k) {
  if (k >= 1)
    g_wait_vm<6>();
  else
    g_wait_vm<0>();
}

__device__ __forceinline__ void g_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((0x3 << 14) | 0xF | (0x7 << 4));
}

// Six 1 KB DMA instructions: instruction i reads from the wave-uniform base
// b[i] plus this lane's offset off[i] into LDS m0 = lds_addr + 1 KB i (lane l's
// 16 bytes at m0 + 16 l).  The kernel counts these loads itself (vmcnt) and
// orders the slabs with s_barrier.
__device__ __forceinline__ void g_dma6(const unsigned char* const b[6], const uint32_t off[6],
                                       uint32_t lds_addr) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %13\n\tglobal_load_lds_dwordx4 %1, %7\n\t"
      "s_mov_b32 m0, %14\n\tglobal_load_lds_dwordx4 %2, %8\n\t"
      "s_mov_b32 m0, %15\n\tglobal_load_lds_dwordx4 %3, %9\n\t"
      "s_mov_b32 m0, %16\n\tglobal_load_lds_dwordx4 %4, %10\n\t"
      "s_mov_b32 m0, %17\n\tglobal_load_lds_dwordx4 %5, %11\n\t"
      "s_mov_b32 m0, %18\n\tglobal_load_lds_dwordx4 %6, %12\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "v"(off[5]),
        "s"(b[0]), "s"(b[1]), "s"(b[2]), "s"(b[3]), "s"(b[4]), "s"(b[5]),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 1024)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 2048)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 3072)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 4096)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 5120))
      : "memory");
}

__device__ __forceinline__ f32x4 g_mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

struct GhostGrid {
  int nS, ntb, nsup;  // S blocks, t blocks, super-tiles per sample
};

__host__ __device__ inline GhostGrid ghost_grid(int T) {
  GhostGrid g;
  g.nS = (T + kGs - 1) / kGs;
  g.ntb = T / kGt;
  const int nI = (g.nS + kSupS - 1) / kSupS;  // = ceil(ntb / kSupT)
  g.nsup = nI * (nI + 1) / 2;
  return g;
}

// Tiles (S, t) of one sample with t >= 2 S, counted row by row.
__host__ __device__ inline int ghost_ntiles(const GhostGrid& g) { return g.nS * g.ntb - g.nS * (g.nS - 1); }

__global__ void __launch_bounds__(512, 1) k_ghost_mfma(const bf16_t* __restrict__ A,
                                                       const bf16_t* __restrict__ G, int B, int T,
                                                       int d, int p, double* __restrict__ part) {
  __shared__ double red[8];
  const GhostGrid gg = ghost_grid(T);
  // workgroup -> (super-tile, position): round r of XCD x holds super-tile 8 r + x
  const int w = blockIdx.x;
  const int xi = w / kXcd;
  const int sup_all = (xi / 32) * kXcd + w % kXcd;
  if (sup_all >= B * gg.nsup) return;
  const int b = sup_all / gg.nsup;
  int rem = sup_all - b * gg.nsup, I = 0;
  const int nI = (gg.nS + kSupS - 1) / kSupS;
  while (rem >= nI - I) {
    rem -= nI - I;
    ++I;
  }
  const int J = I + rem;
  const int pos = xi % 32;
  const int S = kSupS * I + pos / kSupT, tb = kSupT * J + pos % kSupT;
  if (S >= gg.nS || tb >= gg.ntb || tb < 2 * S) return;  // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nA = d / kGk, n = nA + p / kGk;
  const int64_t row0 = static_cast<int64_t>(b) * T;

  // DMA: wave w fills LDS rows 48 w .. 48 w + 47 (six 8-row blocks q = 6 w + i;
  // blocks 0-31 are the S rows, 32-47 the t rows); lane l -> row l / 8 of the
  // block, LDS chunk l % 8, which holds global chunk (l % 8) ^ g_swz(row): each
  // row's 128 bytes of a slab are one cache line.  S rows past T read row T - 1
  // (block base and lane row both clamped).
  const unsigned char* gb[6];
  uint32_t goff[6];
  const int lr = lane >> 3;
  const int gcol = ((lane & 7) ^ g_swz(lr)) * 8;
  auto phase = [&](const bf16_t* X, int K) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int q = 6 * wave + i;
      int br, lrow;
      if (q < 32) {
        const int t0 = kGs * S + 8 * q;
        br = t0 < T ? t0 : T - 1;
        lrow = (t0 + lr < T ? t0 + lr : T - 1) - br;
      } else {
        br = kGt * tb + 8 * (q - 32);
        lrow = lr;
      }
      gb[i] = reinterpret_cast<const unsigned char*>(X + (row0 + br) * K);
      goff[i] = static_cast<uint32_t>((lrow * K + gcol) * 2);
    }
  };
  const uint32_t lds0 = g_lds_addr(g_lds) + 6 * 1024 * wave;
  auto issue = [&](int s) {
    if (s == 0) phase(A, d);
    if (s == nA) phase(G, p);
    g_dma6(gb, goff, lds0 + (s % kGStages) * kGStage);
#pragma unroll
    for (int i = 0; i < 6; ++i) gb[i] += kGRow;
  };

  // Operand reads: wave (ws, wt) = (w / 2, w % 2) owns S rows 64 ws .. + 63 and t
  // rows 64 wt .. + 63; fragment mb (nb) of k-step h of a slab is rows
  // 16 mb + (l % 16) of that range, chunk 4 h + g with g = l / 16 (feature slots
  // 8 g .. 8 g + 7 of the k-step).  The swizzle depends on l % 16 only: one base
  // per operand and k-step, the blocks 2 KB apart.
  const int ws = wave >> 1, wt = wave & 1;
  const int li = lane & 15, g = lane >> 4;
  const int rd_s0 = (64 * ws + li) * kGRow + ((g ^ g_swz(li)) << 4);
  const int rd_t0 = (kGs + 64 * wt + li) * kGRow + ((g ^ g_swz(li)) << 4);
  const int rd_s1 = (64 * ws + li) * kGRow + (((4 + g) ^ g_swz(li)) << 4);
  const int rd_t1 = (kGs + 64 * wt + li) * kGRow + (((4 + g) ^ g_swz(li)) << 4);

  struct Frag {
    u32x4 s[4], t[4];
  };
  // fragments r0 .. r1 - 1 of the 8 (4 of S, then 4 of t) of k-step h of slab st
  auto read_frags = [&](int st, int h, Frag& f, int r0, int r1) {
    const unsigned char* base = g_lds + (st % kGStages) * kGStage;
    const int os = h ? rd_s1 : rd_s0, ot = h ? rd_t1 : rd_t0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r < r0 || r >= r1) continue;
      if (r < 4)
        f.s[r] = *(g_lds_u32x4*)(base + os + r * 16 * kGRow);
      else
        f.t[r - 4] = *(g_lds_u32x4*)(base + ot + (r - 4) * 16 * kGRow);
    }
  };
  f32x4 ga[4][4], gg2[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ga[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      gg2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  auto mma = [&](const Frag& f, f32x4 (&acc)[4][4], int m0, int m1) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m < m0 || m >= m1) continue;
      acc[m >> 2][m & 3] = g_mfma(f.s[m >> 2], f.t[m & 3], acc[m >> 2][m & 3]);
    }
  };
  auto interleave = [&](int pairs) {
#pragma unroll
    for (int k = 0; k < pairs; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
  };

  // Prologue: slabs 0 and 1 in flight; once slab 0 has landed everywhere the
  // operands of its first k-step go to registers and slab 2 fills the third slot.
  issue(0);
  if (n > 1) issue(1);
  g_wait_slabs(n > 1 ? 1 : 0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  Frag F0, F1;
  read_frags(0, 0, F0, 0, 8);
  if (n > 2) issue(2);

  // Slab s (the operands of its first k-step in F0): the second k-step's
  // operands are read under the first k-step's products.  Then this wave waits
  // for its loads of slab s + 1 and its reads of slab s; after the barrier slab
  // s + 1 has landed for every wave and no wave reads slab s's slot, which takes
  // slab s + 3.  The first k-step of slab s + 1 is read under the second k-step's
  // products.
  auto slab = [&](int s, f32x4 (&acc)[4][4]) {
    read_frags(s, 1, F1, 0, 8);
    mma(F0, acc, 0, 16);
    interleave(8);
    g_wait_slabs(n - 2 - s);
    g_wait_lgkm0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // unconditional, so that reads and products share one basic block: after the
    // last slab this reads a slot no later slab fills, unused
    read_frags(s + 1, 0, F0, 0, 4);
    mma(F1, acc, 0, 8);
    interleave(4);
    if (s + kGStages < n) issue(s + kGStages);
    read_frags(s + 1, 0, F0, 4, 8);
    mma(F1, acc, 8, 16);
    interleave(4);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };
  for (int s = 0; s < nA; ++s) slab(s, ga);
  for (int s = nA; s < n; ++s) slab(s, gg2);

  // Lane (li, g) holds element (4 g + r, li) of block (mb, nb): S token
  // 256 S + 64 ws + 16 mb + 4 g + r, t token 128 tb + 64 wt + 16 nb + li.
  double acc = 0.0;
  if (tb >= 2 * S + 2) {  // wholly above the diagonal: weight 2 (applied below)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc += static_cast<double>(ga[i][j][r]) * static_cast<double>(gg2[i][j][r]);
    acc *= 2.0;
  } else {
    const int sbase = kGs * S + 64 * ws + 4 * g, tbase = kGt * tb + 64 * wt + li;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sv = sbase + 16 * i + r, tv = tbase + 16 * j;
          const double wgt = sv < tv ? 2.0 : (sv == tv ? 1.0 : 0.0);
          acc += wgt * static_cast<double>(ga[i][j][r]) * static_cast<double>(gg2[i][j][r]);
        }
  }
  acc = wave_sum_d(acc);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) tot += red[i];
    const int idx = S * gg.ntb - S * (S - 1) + (tb - 2 * S);
    part[static_cast<int64_t>(b) * ghost_ntiles(gg) + idx] = tot;
  }
}

}  // namespace

bool mfma_ghost_ok(int T, int d, int p) {
  return T > 0 && T % kGt == 0 && d > 0 && d % kGk == 0 && p > 0 && p % kGk == 0 &&
         static_cast<int64_t>(d) * 8 * 2 < (int64_t{1} << 31) &&
         static_cast<int64_t>(p) * 8 * 2 < (int64_t{1} << 31);
}

int mfma_ghost_nparts(int T) { return ghost_ntiles(ghost_grid(T)); }

hipError_t launch_ghost_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p,
                             double* part, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!mfma_ghost_ok(T, d, p)) return hipErrorInvalidValue;
  const GhostGrid gg = ghost_grid(T);
  const int64_t rounds = (static_cast<int64_t>(B) * gg.nsup + kXcd - 1) / kXcd;
  const int64_t nwg = rounds * kXcd * 32;
  if (nwg > (int64_t{1} << 31) - 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_ghost_mfma, dim3(static_cast<unsigned>(nwg)), dim3(512), 0, s, A, G, B, T,
                     d, p, part);
  return hipGetLastError();
}

}  // namespace dprc
