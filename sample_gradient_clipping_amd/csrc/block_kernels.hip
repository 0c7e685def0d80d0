// Forward pass and backward pass 1 of a Llama MLP block on gfx950 (the
// randomized-clipping summary, section アルゴリズム的フロー, steps 1 and 2:
// activations, then every layer's per-sample output gradient).
//
//   RMSNorm   rstd = 1 / sqrt(mean(x^2) + eps), xhat = x rstd, y = gamma xhat
//   linears   g = y Wg^T, u = y Wu^T, out = x + h Wd^T           (NT products)
//   SwiGLU    h = silu(g) u
//   backward  dh = R Wd, (dg, du) from dh, dy = dg Wg + du Wu,
//             dx = rstd (gamma dy - xhat mean(gamma dy xhat)) + R
//
// The products are NT: C[m][n] = sum_k A[m][k] B[n][k] with both operands
// contiguous along k, activations token-major and weights in their [out][in]
// layout; the backward-data products take the transposed bf16 weight copy, so
// they are NT too.
//
// NT GEMM data path.  A workgroup computes a 256 x 256 tile with eight waves of
// 128 (m) x 64 (n).  Stages of 32 k go from HBM into LDS with global_load_lds
// (16 bytes a lane, no registers), four stages, three in flight.  In LDS a
// stage holds 256 rows of 64 bytes per operand; the four 16-byte chunks of row
// r sit in the order c ^ s(r), s(r) = (r >> 1) & 3.  Measured with a probe of
// the operand reads alone, this takes 5.2 cycles per 16-byte read instruction
// per wave against 8.7 with no swizzle (and with ((r >> 1) ^ (r >> 3)) & 3,
// which looked conflict-free on paper).  The DMA writes 1 KB of consecutive LDS
// per instruction, so the swizzle is applied on the global side: the lane that
// fills LDS chunk c of row r fetches global chunk c ^ s(r).  v_mfma_f32_16x16x32_bf16 takes the
// weight fragment as its first operand, so that each lane's four accumulator
// registers are four consecutive n of one m: one 8-byte bf16 store.
//
// SwiGLU lives in the products' epilogues.  Forward: gate and up are one product
// whose weight side alternates 16-row blocks of Wg and Wu, so a wave's 64
// output columns are g, u, g, u blocks of the same hidden columns and each lane
// holds g and u of the same four outputs: it writes g, u and h = silu(g) u.
// Backward: the product dh = R Wd turns into dL/dg = dh u silu'(g) and
// dL/du = dh silu(g) in its epilogue, reading the stored g and u; dh itself
// never goes to memory.
#include "common.h"
#include "internal.h"

namespace dprc {
namespace {

constexpr int kNtM = 256, kNtN = 256, kNtK = 32;
constexpr int kNtRowBytes = kNtK * 2;                 // 64
constexpr int kNtSideBytes = kNtM * kNtRowBytes;      // 16 KB
constexpr int kNtStageBytes = 2 * kNtSideBytes;       // A side, then B side
constexpr int kNtWaves = 8;

__shared__ __attribute__((aligned(16))) unsigned char nt_lds0[kNtStageBytes];
__shared__ __attribute__((aligned(16))) unsigned char nt_lds1[kNtStageBytes];
__shared__ __attribute__((aligned(16))) unsigned char nt_lds2[kNtStageBytes];
__shared__ __attribute__((aligned(16))) unsigned char nt_lds3[kNtStageBytes];

typedef __attribute__((address_space(3))) void nt_lds_void;
typedef __attribute__((address_space(3))) const u32x4 nt_lds_u32x4;

__device__ __forceinline__ u32x4 nt_read16(const unsigned char* p) {
  return *(nt_lds_u32x4*)(p);
}

template <int N>
__device__ __forceinline__ void nt_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): the wave's LDS reads (and scalar loads) have returned;
// vmcnt and expcnt unconstrained.
__device__ __forceinline__ void nt_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((0x3 << 14) | 0xF | (0x7 << 4));
}

__device__ __forceinline__ uint32_t nt_lds_addr(const unsigned char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((nt_lds_void*)(p)));
}

__host__ __device__ __forceinline__ int nt_swz(int r) { return (r >> 1) & 3; }

// One 1 KB DMA instruction: lane i's 16 global bytes land at LDS m0 + 16 i.
// m0 is saved and restored around the load (the compiler keeps its own value
// there).  The kernel counts these loads itself (vmcnt) and orders stages with
// s_barrier; as inline asm they are not LDS writes the compiler would drain
// before every LDS read.
__device__ __forceinline__ void nt_dma(const unsigned char* gp, uint32_t lds_addr) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(gp), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}

// Four 1 KB DMA instructions of one stage: instruction i reads from the
// wave-uniform base b[i] (SGPRs) plus this lane's 32-bit offset off[i], into
// LDS m0 = lds_addr + 1 KB i.  No per-load address arithmetic.
__device__ __forceinline__ void nt_dma4(const unsigned char* const b[4], const uint32_t off[4],
                                        uint32_t lds_addr) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %9\n\tglobal_load_lds_dwordx4 %1, %5\n\t"
      "s_mov_b32 m0, %10\n\tglobal_load_lds_dwordx4 %2, %6\n\t"
      "s_mov_b32 m0, %11\n\tglobal_load_lds_dwordx4 %3, %7\n\t"
      "s_mov_b32 m0, %12\n\tglobal_load_lds_dwordx4 %4, %8\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(b[0]), "s"(b[1]), "s"(b[2]),
        "s"(b[3]), "s"(__builtin_amdgcn_readfirstlane(lds_addr)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 1024)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 2048)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 3072))
      : "memory");
}

__device__ __forceinline__ f32x4 nt_mfma(u32x4 w, u32x4 x, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                 __builtin_bit_cast(bf16x8, x), c, 0, 0, 0);
}

// Workgroup -> (m tile, n tile): the eight XCDs (consecutive workgroups go to
// them in turn) each get a contiguous run of the logical order, which walks n
// inside groups of four m tiles.
__device__ __forceinline__ void nt_tile_of(int w, int tm, int tn, int nwg, int& mt, int& nt) {
  constexpr int kXcd = 8, kGroupM = 4;
  const int l = (nwg % kXcd == 0) ? (w % kXcd) * (nwg / kXcd) + w / kXcd : w;
  const int grp = l / (kGroupM * tn);
  const int r = l - grp * kGroupM * tn;
  const int gm = tm - grp * kGroupM < kGroupM ? tm - grp * kGroupM : kGroupM;
  nt = r / gm;
  mt = grp * kGroupM + (r - nt * gm);
}

constexpr int kEpiStore = 0, kEpiResid = 1, kEpiSwiglu = 2, kEpiSwigluBwd = 3;

__device__ __forceinline__ float nt_sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

struct NtArgs {
  const bf16_t* A1;
  const bf16_t* B1;
  const bf16_t* B1u;  // kEpiSwiglu: the up weight
  const bf16_t* A2;
  const bf16_t* B2;
  const bf16_t* A3;
  const bf16_t* B3;
  const bf16_t* Rz;   // kEpiResid: residual; kEpiSwigluBwd: g
  const bf16_t* Rz2;  // kEpiSwigluBwd: u
  bf16_t* C;
  bf16_t* C2;
  bf16_t* C3;
  int K1, K2, K3, M, N;
};

// acc[m][n] = sum_k A1[m][k] B1[n][k] + sum_k A2[m][k] B2[n][k] + sum_k A3[m][k] B3[n][k],
// then by EPI:
//   kEpiStore   C = bf16(acc)
//   kEpiResid   C = bf16(acc + Rz)
//   kEpiSwiglu  weight rows alternate 16-row blocks of B1 (gate) and B1u (up);
//               C = g, C2 = u, C3 = h = silu(g) u, each [M][N / 2]
//   kEpiSwigluBwd  acc = dh; C = dh u silu'(g), C2 = dh silu(g), with g = Rz,
//               u = Rz2 ([M][N])
// K1, K2, K3 multiples of 32 (K2, K3 may be 0), N a multiple of 256, any M >= 1: rows
// of A beyond M are read from row M - 1 and their results not stored.
template <int EPI>
__global__ void __launch_bounds__(512, 1) k_gemm_nt(const NtArgs a) {
  const bf16_t* __restrict__ A1 = a.A1;
  const bf16_t* __restrict__ A2 = a.A2;
  const int K1 = a.K1, K2 = a.K2, K3 = a.K3, M = a.M, N = a.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int mt, ntile;
  nt_tile_of(blockIdx.x, (M + kNtM - 1) / kNtM, N / kNtN, gridDim.x, mt, ntile);
  const int m0 = mt * kNtM, n0 = ntile * kNtN;
  const int ns1 = K1 / kNtK;
  const int ns12 = ns1 + K2 / kNtK;
  const int nstage = ns12 + K3 / kNtK;

  // DMA: wave w fills rows (w & 3) * 64 .. + 63 of side w >> 2 (0: A, 1: B),
  // 16 rows per instruction; lane i -> row i / 4, LDS chunk i % 4.
  const int side = wave >> 2;
  const int rbase = (wave & 3) * 64;
  const int dst_off = side * kNtSideBytes + rbase * kNtRowBytes;
  const int r0 = rbase + (lane >> 2);
  // Instruction i covers rows 16 i + rbase / 16 ..; rbase / 16 is even, so the
  // 16-row block of instruction i is a gate block for even i, an up block for odd.
  const bf16_t* src1[2] = {side == 0 ? A1 : a.B1,
                           side == 0 ? A1 : (EPI == kEpiSwiglu ? a.B1u : a.B1)};
  const bf16_t* src2 = side == 0 ? A2 : a.B2;
  const bf16_t* src3 = side == 0 ? a.A3 : a.B3;

  // Instruction i loads a 16-row block through a wave-uniform base that
  // advances 64 bytes per stage; each lane adds its row and chunk offset (both
  // re-formed when the k range moves to the next operand pair).  On the A side
  // rows past M read row M - 1: the block's base row is clamped to M - 1 and
  // each lane's row to M - 1, so the lane offset is never negative.  On the
  // interleaved gate/up side, block i is block (rbase / 32 + i / 2) of the gate
  // rows for even i and of the up rows for odd i.
  const unsigned char* gb[4];
  uint32_t goff[4];
  auto phase = [&](const bf16_t* sa, const bf16_t* sb, int K) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int br, lrow;
      if (side == 0) {
        const int b0 = m0 + rbase + 16 * i;
        br = b0 < M ? b0 : M - 1;
        lrow = (b0 + (lane >> 2) < M ? b0 + (lane >> 2) : M - 1) - br;
      } else {
        br = EPI == kEpiSwiglu ? n0 / 2 + ((rbase >> 5) + (i >> 1)) * 16 : n0 + rbase + 16 * i;
        lrow = lane >> 2;
      }
      gb[i] = reinterpret_cast<const unsigned char*>((i & 1 ? sb : sa) + static_cast<int64_t>(br) * K);
      const int gcol = ((lane & 3) ^ nt_swz(r0)) * 8;  // the same for every 16-row block
      goff[i] = static_cast<uint32_t>((lrow * K + gcol) * 2);
    }
  };
  auto issue = [&](int s, unsigned char* stage_lds) {
    if (s == 0)
      phase(src1[0], src1[1], K1);
    else if (s == ns1)
      phase(src2, src2, K2);
    else if (s == ns12)
      phase(src3, src3, K3);
    nt_dma4(gb, goff, nt_lds_addr(stage_lds) + dst_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) gb[i] += kNtK * 2;
  };

  // Operand reads: wave tile rows wm * 128 + mb * 16 + (lane % 16) of A and
  // wn * 64 + nb * 16 + (lane % 16) of B, chunk g = lane / 16 of each (k slots
  // 8 g .. 8 g + 7 for both operands).
  const int wm = wave >> 2, wn = wave & 3;
  const int li = lane & 15, g = lane >> 4;
  // The swizzle of row r = base + 16 mb + li depends on li only: one base
  // address per operand, the blocks at constant offsets from it.
  const int ra = wm * 128 + li, rb = wn * 64 + li;
  const int rd_a = ra * kNtRowBytes + ((g ^ nt_swz(ra)) << 4);
  const int rd_b = kNtSideBytes + rb * kNtRowBytes + ((g ^ nt_swz(rb)) << 4);

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A stage's MFMA operands, read from LDS into registers one stage ahead of
  // the products that use them.
  struct Frag {
    u32x4 xa[8], wb[4];
  };
  // reads r0 .. r1 - 1 of the 12 (the 4 weight fragments, then the 8 of A)
  auto read_frags = [&](const unsigned char* st, Frag& f, int r0, int r1) {
#pragma unroll
    for (int r = 0; r < 12; ++r) {
      if (r < r0 || r >= r1) continue;
      if (r < 4)
        f.wb[r] = nt_read16(st + rd_b + r * 16 * kNtRowBytes);
      else
        f.xa[r - 4] = nt_read16(st + rd_a + (r - 4) * 16 * kNtRowBytes);
    }
  };
  // products m0 .. m1 - 1 of the 32 (row block mb = m / 4, column block nb = m % 4)
  auto mma = [&](const Frag& f, int m0_, int m1_) {
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      if (m < m0_ || m >= m1_) continue;
      acc[m >> 2][m & 3] = nt_mfma(f.wb[m & 3], f.xa[m >> 2], acc[m >> 2][m & 3]);
    }
  };

  unsigned char* L0 = nt_lds0;
  unsigned char* L1 = nt_lds1;
  unsigned char* L2 = nt_lds2;
  unsigned char* L3 = nt_lds3;
  Frag F0, F1;

  // Prologue: stages 0..2 in flight; once stage 0 has landed everywhere, its
  // operands go to registers and stage 3 fills the fourth slot.
  if (nstage > 0) issue(0, L0);
  if (nstage > 1) issue(1, L1);
  if (nstage > 2) issue(2, L2);
  if (nstage > 2)
    nt_wait_vm<8>();
  else if (nstage > 1)
    nt_wait_vm<4>();
  else
    nt_wait_vm<0>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (nstage > 0) read_frags(L0, F0, 0, 12);
  if (nstage > 3) issue(3, L3);

  // Step s (stage s's operands are in `cur`): wait for this wave's loads of
  // stage s + 1 (those of s + 2 and s + 3 may stay in flight) and for its LDS
  // reads of stage s; the barrier then certifies that stage s + 1 has landed
  // for every wave and that no wave still reads stage s's slot, which is
  // refilled with stage s + 4.  Stage s + 1's operands are read while stage
  // s's products run, one 16-byte read after every second of the first 24
  // products, so that the reads issue under the matrix pipe instead of ahead
  // of it.
  auto step = [&](int s, const Frag& cur, Frag& next, const unsigned char* next_lds,
                  unsigned char* refill) {
    const int ahead = nstage - 2 - s;  // stages issued beyond s + 1
    if (ahead >= 2)
      nt_wait_vm<8>();
    else if (ahead == 1)
      nt_wait_vm<4>();
    else
      nt_wait_vm<0>();
    nt_wait_lgkm0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // unconditional, so that the reads and the products share one basic block:
    // after the last stage this reads a slot no later stage fills, unused.  The
    // refill's DMA follows the first eight products: every wave leaves the
    // barrier at once, and what a wave issues before its first MFMA leaves
    // the matrix pipe idle.
    read_frags(next_lds, next, 0, 4);
    mma(cur, 0, 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    if (s + 4 < nstage) issue(s + 4, refill);
    read_frags(next_lds, next, 4, 12);
    mma(cur, 8, 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  for (int s = 0; s < nstage; s += 4) {
    step(s, F0, F1, L1, L0);
    if (s + 1 < nstage) step(s + 1, F1, F0, L2, L1);
    if (s + 2 < nstage) step(s + 2, F0, F1, L3, L2);
    if (s + 3 < nstage) step(s + 3, F1, F0, L0, L3);
  }

  // Epilogue: lane (li, g) holds acc[m][n .. n + 3] of block (mb, nb), m = row
  // li of the block, n = 4 g.
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int m = m0 + wm * 128 + mb * 16 + li;
    if (m >= M) continue;
    if constexpr (EPI == kEpiSwiglu) {
      // blocks nb = 0, 1 (and 2, 3) are gate and up of the same 16 hidden columns
      const int F = N / 2;
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int col = n0 / 2 + wn * 32 + pr * 16 + 4 * g;
        const int64_t off = static_cast<int64_t>(m) * F + col;
        const f32x4 gv = acc[mb][2 * pr], uv = acc[mb][2 * pr + 1];
        float h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = gv[e] * nt_sigmoid(gv[e]) * uv[e];
        *reinterpret_cast<uint2*>(a.C + off) = uint2{pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
        *reinterpret_cast<uint2*>(a.C2 + off) = uint2{pack_bf16x2(uv[0], uv[1]), pack_bf16x2(uv[2], uv[3])};
        *reinterpret_cast<uint2*>(a.C3 + off) = uint2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = n0 + wn * 64 + nb * 16 + 4 * g;
        const int64_t off = static_cast<int64_t>(m) * N + n;
        f32x4 v = acc[mb][nb];
        if constexpr (EPI == kEpiSwigluBwd) {
          const uint2 gr = *reinterpret_cast<const uint2*>(a.Rz + off);
          const uint2 ur = *reinterpret_cast<const uint2*>(a.Rz2 + off);
          const float gf[4] = {__uint_as_float(gr.x << 16), __uint_as_float(gr.x & 0xFFFF0000u),
                               __uint_as_float(gr.y << 16), __uint_as_float(gr.y & 0xFFFF0000u)};
          const float uf[4] = {__uint_as_float(ur.x << 16), __uint_as_float(ur.x & 0xFFFF0000u),
                               __uint_as_float(ur.y << 16), __uint_as_float(ur.y & 0xFFFF0000u)};
          float dg[4], du[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sg = nt_sigmoid(gf[e]);
            dg[e] = v[e] * uf[e] * sg * (1.0f + gf[e] * (1.0f - sg));
            du[e] = v[e] * gf[e] * sg;
          }
          *reinterpret_cast<uint2*>(a.C + off) = uint2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
          *reinterpret_cast<uint2*>(a.C2 + off) = uint2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
        } else {
          if constexpr (EPI == kEpiResid) {
            const uint2 r = *reinterpret_cast<const uint2*>(a.Rz + off);
            v[0] += __uint_as_float(r.x << 16);
            v[1] += __uint_as_float(r.x & 0xFFFF0000u);
            v[2] += __uint_as_float(r.y << 16);
            v[3] += __uint_as_float(r.y & 0xFFFF0000u);
          }
          *reinterpret_cast<uint2*>(a.C + off) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Elementwise and row kernels.  Rows are token rows of width d (d % 8 == 0);
// one wave per row, 16-byte accesses (8 bf16 a lane).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack8(u32x4 v, float f[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float f[8]) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

constexpr int kRowWaves = 4;  // rows per 256-thread block

__global__ void __launch_bounds__(256) k_rmsnorm_fwd(const bf16_t* __restrict__ x,
                                                     const float* __restrict__ gamma, int M, int d,
                                                     float eps, bf16_t* __restrict__ xhat,
                                                     bf16_t* __restrict__ y,
                                                     float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const bf16_t* xr = x + row * d;
  const int nc = d >> 3;
  float ss = 0.f;
  for (int c = lane; c < nc; c += 64) {
    float f[8];
    unpack8(*reinterpret_cast<const u32x4*>(xr + 8 * c), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += f[i] * f[i];
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
  if (lane == 0) rstd[row] = rs;
  for (int c = lane; c < nc; c += 64) {
    float f[8], yv[8];
    unpack8(*reinterpret_cast<const u32x4*>(xr + 8 * c), f);
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * c);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * c + 4);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f[i] *= rs;
      yv[i] = gv[i] * f[i];
    }
    *reinterpret_cast<u32x4*>(xhat + row * d + 8 * c) = pack8(f);
    *reinterpret_cast<u32x4*>(y + row * d + 8 * c) = pack8(yv);
  }
}

__global__ void __launch_bounds__(256) k_rmsnorm_bwd(const bf16_t* __restrict__ x,
                                                     const float* __restrict__ rstd,
                                                     const float* __restrict__ gamma,
                                                     const bf16_t* __restrict__ dy,
                                                     const bf16_t* __restrict__ dout, int M, int d,
                                                     bf16_t* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const float rs = rstd[row];
  const int nc = d >> 3;
  float dot = 0.f;  // sum_q gamma dy xhat
  for (int c = lane; c < nc; c += 64) {
    float xf[8], df[8];
    unpack8(*reinterpret_cast<const u32x4*>(x + row * d + 8 * c), xf);
    unpack8(*reinterpret_cast<const u32x4*>(dy + row * d + 8 * c), df);
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * c);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * c + 4);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) dot += gv[i] * df[i] * (xf[i] * rs);
  }
  const float mean = wave_sum(dot) / static_cast<float>(d);
  for (int c = lane; c < nc; c += 64) {
    float xf[8], df[8], rf[8], o[8];
    unpack8(*reinterpret_cast<const u32x4*>(x + row * d + 8 * c), xf);
    unpack8(*reinterpret_cast<const u32x4*>(dy + row * d + 8 * c), df);
    unpack8(*reinterpret_cast<const u32x4*>(dout + row * d + 8 * c), rf);
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * c);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * c + 4);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = rs * (gv[i] * df[i] - xf[i] * rs * mean) + rf[i];
    *reinterpret_cast<u32x4*>(dx + row * d + 8 * c) = pack8(o);
  }
}

// theta fp32 [p][d] -> W bf16 [p][d] and Wt bf16 [d][p], 64 x 64 tiles through
// LDS (p, d multiples of 64).
__global__ void __launch_bounds__(256) k_cast_transpose(const float* __restrict__ theta, int p,
                                                        int d, bf16_t* __restrict__ W,
                                                        bf16_t* __restrict__ Wt) {
  __shared__ bf16_t tile[64][64 + 2];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tr = threadIdx.x >> 4, tc = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = tr + 16 * k;
    const float4 v = *reinterpret_cast<const float4*>(theta + static_cast<int64_t>(r0 + r) * d + c0 + tc);
    uint2 o;
    o.x = pack_bf16x2(v.x, v.y);
    o.y = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<uint2*>(W + static_cast<int64_t>(r0 + r) * d + c0 + tc) = o;
    tile[r][tc + 0] = static_cast<bf16_t>(o.x & 0xFFFFu);
    tile[r][tc + 1] = static_cast<bf16_t>(o.x >> 16);
    tile[r][tc + 2] = static_cast<bf16_t>(o.y & 0xFFFFu);
    tile[r][tc + 3] = static_cast<bf16_t>(o.y >> 16);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = tr + 16 * k;  // column of theta = row of Wt
    uint2 o;
    o.x = static_cast<uint32_t>(tile[tc + 0][c]) | (static_cast<uint32_t>(tile[tc + 1][c]) << 16);
    o.y = static_cast<uint32_t>(tile[tc + 2][c]) | (static_cast<uint32_t>(tile[tc + 3][c]) << 16);
    *reinterpret_cast<uint2*>(Wt + static_cast<int64_t>(c0 + c) * p + r0 + tc) = o;
  }
}

int elementwise_blocks(int64_t n8) {
  const int64_t want = (n8 + 255) / 256;
  return static_cast<int>(want < 4096 ? (want > 0 ? want : 1) : 4096);
}

}  // namespace

bool gemm_nt_ok(int64_t M, int N, int K1, int K2, int K3) {
  // K < 2^26: a lane's byte offset inside its 16-row block, 2 (15 K + 24), fits
  // 32 bits
  constexpr int kKMax = 1 << 26;
  if (K1 >= kKMax || K2 >= kKMax || K3 >= kKMax) return false;
  return M >= 1 && M <= (int64_t{1} << 30) && N > 0 && N % kNtN == 0 && K1 > 0 &&
         K1 % kNtK == 0 && K2 >= 0 && K2 % kNtK == 0 && K3 >= 0 && K3 % kNtK == 0 &&
         (K3 == 0 || K2 > 0);
}

static hipError_t launch_nt(const NtArgs& a, int epi, hipStream_t s) {
  const int64_t tiles = ((static_cast<int64_t>(a.M) + kNtM - 1) / kNtM) * (a.N / kNtN);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(tiles)), block(64 * kNtWaves);
  switch (epi) {
    case kEpiStore: hipLaunchKernelGGL(k_gemm_nt<kEpiStore>, grid, block, 0, s, a); break;
    case kEpiResid: hipLaunchKernelGGL(k_gemm_nt<kEpiResid>, grid, block, 0, s, a); break;
    case kEpiSwiglu: hipLaunchKernelGGL(k_gemm_nt<kEpiSwiglu>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(k_gemm_nt<kEpiSwigluBwd>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const bf16_t* A1, const bf16_t* B1, int K1, const bf16_t* A2,
                          const bf16_t* B2, int K2, int64_t M, int N, const bf16_t* Rz, bf16_t* C,
                          hipStream_t s) {
  return launch_gemm_nt3(A1, B1, K1, A2, B2, K2, nullptr, nullptr, 0, M, N, Rz, C, s);
}

hipError_t launch_gemm_nt3(const bf16_t* A1, const bf16_t* B1, int K1, const bf16_t* A2,
                           const bf16_t* B2, int K2, const bf16_t* A3, const bf16_t* B3, int K3,
                           int64_t M, int N, const bf16_t* Rz, bf16_t* C, hipStream_t s) {
  if (!gemm_nt_ok(M, N, K1, K2, K3)) return hipErrorInvalidValue;
  NtArgs a{};
  a.A1 = A1; a.B1 = B1; a.A2 = A2; a.B2 = B2; a.A3 = A3; a.B3 = B3; a.Rz = Rz; a.C = C;
  a.K1 = K1; a.K2 = K2; a.K3 = K3; a.M = static_cast<int>(M); a.N = N;
  return launch_nt(a, Rz ? kEpiResid : kEpiStore, s);
}

hipError_t launch_gemm_nt_swiglu(const bf16_t* y, const bf16_t* Wg, const bf16_t* Wu, int d,
                                 int64_t M, int f, bf16_t* g, bf16_t* u, bf16_t* h, hipStream_t s) {
  if (f % (kNtN / 2) != 0 || !gemm_nt_ok(M, 2 * f, d, 0, 0)) return hipErrorInvalidValue;
  NtArgs a{};
  a.A1 = y; a.B1 = Wg; a.B1u = Wu; a.C = g; a.C2 = u; a.C3 = h;
  a.K1 = d; a.K2 = 0; a.M = static_cast<int>(M); a.N = 2 * f;
  return launch_nt(a, kEpiSwiglu, s);
}

hipError_t launch_gemm_nt_swiglu_bwd(const bf16_t* dout, const bf16_t* WdT, int d, int64_t M, int f,
                                     const bf16_t* g, const bf16_t* u, bf16_t* dg, bf16_t* du,
                                     hipStream_t s) {
  if (!gemm_nt_ok(M, f, d, 0, 0)) return hipErrorInvalidValue;
  NtArgs a{};
  a.A1 = dout; a.B1 = WdT; a.Rz = g; a.Rz2 = u; a.C = dg; a.C2 = du;
  a.K1 = d; a.K2 = 0; a.M = static_cast<int>(M); a.N = f;
  return launch_nt(a, kEpiSwigluBwd, s);
}

hipError_t launch_rmsnorm_fwd(const bf16_t* x, const float* gamma, int64_t M, int d, float eps,
                              bf16_t* xhat, bf16_t* y, float* rstd, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d <= 0 || d % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rmsnorm_fwd, dim3(static_cast<unsigned>((M + kRowWaves - 1) / kRowWaves)),
                     dim3(256), 0, s, x, gamma, static_cast<int>(M), d, eps, xhat, y, rstd);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const bf16_t* x, const float* rstd, const float* gamma,
                              const bf16_t* dy, const bf16_t* dout, int64_t M, int d, bf16_t* dx,
                              hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d <= 0 || d % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3(static_cast<unsigned>((M + kRowWaves - 1) / kRowWaves)),
                     dim3(256), 0, s, x, rstd, gamma, dy, dout, static_cast<int>(M), d, dx);
  return hipGetLastError();
}

hipError_t launch_cast_transpose(const float* theta, int p, int d, bf16_t* W, bf16_t* Wt,
                                 hipStream_t s) {
  if (p <= 0 || d <= 0) return hipSuccess;
  if (p % 64 != 0 || d % 64 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cast_transpose, dim3(d / 64, p / 64), dim3(256), 0, s, theta, p, d, W, Wt);
  return hipGetLastError();
}

}  // namespace dprc
