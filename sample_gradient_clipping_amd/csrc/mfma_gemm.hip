// MFMA contraction over tokens for bf16 inputs on gfx950:
//   aggregate   part[split][o][q] = sum_{tokens} c_i G_i[t][o] A_i[t][q]
//               (the clipped sum S = sum_i c_i G_i^T A_i: glossary page, section
//               DP-SGDのアルゴリズム, step 4; randomized-clipping summary,
//               section アルゴリズム的フロー, step 5)
//   fgc         M_i[o][q]            = sum_t G_i[t][o] A_i[t][q]   (FGC baseline)
// M = o (p), N = q (d), K = tokens.
//
// Data path.  Both operands are stored token-major, so the contraction index
// is the strided one.  Tiles of 32 tokens go from HBM straight into LDS with
// global_load_lds (no registers, no VALU), in their natural [token][column]
// layout; the MFMA operands then come out of LDS with ds_read_b64_tr_b16,
// which transposes 16-bit values inside each group of 16 lanes: output lane i,
// slot j receives element (i mod 4) of the 8 bytes that lane 4 j + i / 4 of the
// group addressed.  Pointing lane 4 j + q of group g at token row 8 g + 2 j + h,
// columns c0 + 4 q .. + 3, gives lane i the four tokens 8 g + h + {0,2,4,6} of
// column c0 + i -- the v_mfma_f32_16x16x32_bf16 operand layout (lane i: row or
// column i % 16, lane group g: 8 contraction values), two reads (h = 0, 1) per
// operand.  Which token sits in which contraction slot is immaterial as long
// as both operands agree.  One 16-byte DMA instruction fills two consecutive
// 512-byte rows; each such row pair is followed by 32 bytes of padding, so the
// four rows read by a 16-lane group (four different pairs) start 8 banks apart.
//
// Pipeline.  Workgroup tile 256 x 256, eight waves of 128 (M) x 64 (N), four
// LDS stages of 32 tokens.  Each stage lives in its own __shared__ array so
// that the compiler can see the in-flight LDS DMA does not alias the stage
// being read; the loop is unrolled over the four arrays.  A stage's operands
// are read from LDS into registers one step ahead of its products, so the
// transposing reads of stage s+1 run under the MFMAs of stage s, and the slot
// of stage s is refilled (stage s+4) as soon as every wave has read it.
// Synchronisation is an explicit vmcnt wait for this wave's loads plus a bare
// s_barrier (no fence that would drain the loads of later stages).  Inside a
// step the 24 transposing reads are interleaved one by one with the first 24
// of its 32 MFMAs, and the refill's DMA is issued after the first eight of
// them: every wave leaves the barrier at the same moment, and whatever a wave
// issues before its first MFMA leaves the matrix pipe of its SIMD idle.
//
// Per-sample clip factors without a second accumulator: the active samples are
// visited in ascending c, and the accumulator holds sum_{seen} (c_seg / c_cur)
// S_seg.  Entering a sample with factor c_new multiplies it by c_cur / c_new
// (<= 1, so it never overflows); the final tile is multiplied by the last c.
#include "common.h"
#include "internal.h"

namespace dprc {

constexpr int kGM = 256, kGN = 256, kGK = 32;
constexpr int kWaves = 8;
constexpr int kRowBytes = 512;                  // 256 bf16
constexpr int kPairBytes = 2 * kRowBytes + 32;  // two rows + pad
constexpr int kSideBytes = (kGK / 2) * kPairBytes;  // one operand, one stage
constexpr int kStageBytes = 2 * kSideBytes;     // G tile then A tile
constexpr int kNStage = 4;
constexpr int kGroup = kNStage * kGK;           // tokens per unrolled loop trip

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_cvoid;

__shared__ __attribute__((aligned(16))) unsigned char g_lds0[kStageBytes];
__shared__ __attribute__((aligned(16))) unsigned char g_lds1[kStageBytes];
__shared__ __attribute__((aligned(16))) unsigned char g_lds2[kStageBytes];
__shared__ __attribute__((aligned(16))) unsigned char g_lds3[kStageBytes];

// s_waitcnt immediate: vmcnt = N, expcnt and lgkmcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): the wave's LDS reads (and scalar loads) have returned;
// vmcnt and expcnt unconstrained.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((0x3 << 14) | 0xF | (0x7 << 4));
}

__device__ __forceinline__ v4i16 tr_read(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

// Four row pairs (each 64 lanes x 16 bytes = two 512-byte rows) from HBM into
// LDS.  Issued as inline asm so that the compiler does not treat the DMA as an
// LDS write it must drain before every later LDS read: the kernel counts these
// loads itself (wait_vm) and orders the stages with s_barrier.  lds_addr is
// the wave-uniform LDS byte address of the first pair (goes to m0); off[i] is
// this lane's byte offset of pair i from the wave-uniform gbase, so that the
// issue is four m0 writes and four loads, with no 64-bit address arithmetic
// per load (that arithmetic, on the scalar unit after every stage barrier,
// cost 3% of the contraction).
__device__ __forceinline__ void dma_pairs(const unsigned char* gbase, const uint32_t off[4],
                                          uint32_t lds_addr) {
  // m0 carries the LDS address; it is saved and restored around the loads
  // (the compiler reserves m0 and must find it unchanged).  The global address
  // is the wave-uniform base (SGPRs) plus this lane's 32-bit offset.
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\tglobal_load_lds_dwordx4 %1, %5\n\t"
      "s_mov_b32 m0, %7\n\tglobal_load_lds_dwordx4 %2, %5\n\t"
      "s_mov_b32 m0, %8\n\tglobal_load_lds_dwordx4 %3, %5\n\t"
      "s_mov_b32 m0, %9\n\tglobal_load_lds_dwordx4 %4, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(gbase),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + kPairBytes)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 2 * kPairBytes)),
        "s"(__builtin_amdgcn_readfirstlane(lds_addr + 3 * kPairBytes))
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const unsigned char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(p)));
}

__device__ __forceinline__ f32x4 mfma_tr(v4i16 a0, v4i16 a1, v4i16 b0, v4i16 b1, f32x4 c) {
  const v8i16 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  const v8i16 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Workgroup -> (o tile, q tile, split).  Consecutive workgroups go to the
// eight XCDs in turn, each with its own L2; the logical work list is dealt out
// so that every XCD gets a contiguous run of it, and the list is ordered in
// groups of four o tiles (q outer, o inner), so that a run of 32 workgroups
// covers a 4 x 8 block of tiles of one split: 12 distinct operand panels per
// XCD instead of up to 33 with the plain row-major order.
__device__ __forceinline__ int xcd_dealt(int w, int n) {
  constexpr int kXcd = 8;
  return (n % kXcd == 0) ? (w % kXcd) * (n / kXcd) + w / kXcd : w;
}

// Tile t of a to x tq grid in groups of four o tiles (q outer, o inner).
__device__ __forceinline__ void tile_in_grid(int t, int to, int tq, int& ot, int& qt) {
  constexpr int kGroupM = 4;
  const int grp = t / (kGroupM * tq);
  const int r = t - grp * kGroupM * tq;
  const int gm = to - grp * kGroupM < kGroupM ? to - grp * kGroupM : kGroupM;
  qt = r / gm;
  ot = grp * kGroupM + (r - qt * gm);
}

__device__ __forceinline__ void tile_of(int w, int to, int tq, int n, int& ot, int& qt, int& z) {
  const int l = xcd_dealt(w, n);
  const int tiles = to * tq;
  z = l / tiles;
  tile_in_grid(l - z * tiles, to, tq, ot, qt);
}

// One workgroup's tile (o tile ot, q tile qt, token split or sample z).
// MODE 0: clipped aggregation, split-K over the active samples in ascending c.
// MODE 1: FGC, z = sample, whole sample, no scaling.
template <int MODE>
__device__ __forceinline__ void gemm_tile(const bf16_t* __restrict__ A,
                                          const bf16_t* __restrict__ G, int T, int d, int p,
                                          const float* __restrict__ cvec,
                                          const int* __restrict__ order,
                                          const int* __restrict__ count, int64_t split_tokens,
                                          int ot, int qt, int z, float* __restrict__ out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int o0 = ot * kGM;
  const int q0 = qt * kGN;

  // Token range of this workgroup, as positions kv in the visiting order.
  int64_t kv0, kv1;
  if (MODE == 0) {
    const int64_t Kv = static_cast<int64_t>(*count) * T;
    kv0 = static_cast<int64_t>(z) * split_tokens;
    kv1 = kv0 + split_tokens < Kv ? kv0 + split_tokens : Kv;
  } else {
    kv0 = 0;
    kv1 = T;
  }
  const int nstage = kv1 > kv0 ? static_cast<int>((kv1 - kv0) / kGK) : 0;

  // ---- LDS DMA: wave w fills row pairs (w & 3) * 4 .. + 3 (token rows
  // 8 (w & 3) .. + 7) of side w >> 2 (0: G, 1: A); lanes 0-31 take the even
  // row of a pair, lanes 32-63 the odd one, 16 bytes (8 columns) each.
  const int side = wave >> 2;
  const int pair0 = (wave & 3) * 4;
  const bf16_t* src = side == 0 ? G : A;
  const int ld = side == 0 ? p : d;
  const int col0 = side == 0 ? o0 : q0;
  const uint32_t lane_src =
      static_cast<uint32_t>(((2 * pair0 + (lane >> 5)) * ld + col0 + (lane & 31) * 8) * 2);
  const uint32_t pair_step = static_cast<uint32_t>(2 * ld * 2);
  const uint32_t dma_off[4] = {lane_src, lane_src + pair_step, lane_src + 2 * pair_step,
                                lane_src + 3 * pair_step};
  const int dst_off = side * kSideBytes + pair0 * kPairBytes;
  const int64_t stage_bytes_g = static_cast<int64_t>(kGK) * ld * 2;

  // The sample being loaded is looked up once per sample (its entry of the
  // visiting order is read when the previous sample's last tile is issued), so
  // that no stage waits on a scalar load after its barrier.
  int64_t ld_seg = kv0 / T;
  int ld_off = static_cast<int>(kv0 - ld_seg * T);
  const int64_t nseg = MODE == 0 ? static_cast<int64_t>(*count) : 1;
  int64_t ld_sample = MODE == 0 ? (nstage > 0 ? static_cast<int64_t>(order[ld_seg]) : 0)
                                : static_cast<int64_t>(z);
  // wave-uniform global base of the next stage to load, advanced by one stage
  // per issue and re-formed when the visiting order moves to the next sample
  const unsigned char* gbase =
      reinterpret_cast<const unsigned char*>(src + (ld_sample * T + ld_off) * ld);
  auto issue = [&](unsigned char* stage_lds) {
    dma_pairs(gbase, dma_off, lds_addr_of(stage_lds) + dst_off);
    gbase += stage_bytes_g;
    ld_off += kGK;
    if (ld_off == T) {
      ld_off = 0;
      ++ld_seg;
      if (MODE == 0 && ld_seg < nseg) {
        ld_sample = order[ld_seg];
        gbase = reinterpret_cast<const unsigned char*>(src + ld_sample * T * ld);
      }
    }
  };

  // ---- MFMA operand reads.  Wave tile: rows wm*128 .. +128 of M, cols
  // wn*64 .. +64 of N.  Lane 4 j + q of group g addresses token row
  // 8 g + 2 j + h (pair 4 g + j, row h of the pair), columns c0 + 4 q .. + 3.
  const int wm = wave >> 2, wn = wave & 3;
  const int g = lane >> 4, li = lane & 15;
  const int rd_lane = (4 * g + (li >> 2)) * kPairBytes + (li & 3) * 8;
  const int rd_a = rd_lane + wm * 128 * 2;
  const int rd_b = kSideBytes + rd_lane + wn * 64 * 2;

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A stage's MFMA operands, read from LDS into registers one stage ahead of
  // the products that use them.
  struct Frag {
    v4i16 a[8][2], b[4][2];
  };
  // reads r0 .. r1 - 1 of the 24 (16 of the 128-wide operand, then 8)
  auto read_frags = [&](const unsigned char* st, Frag& f, int r0, int r1) {
#pragma unroll
    for (int r = 0; r < 24; ++r) {
      if (r < r0 || r >= r1) continue;
      if (r < 16)
        f.a[r >> 1][r & 1] = tr_read(st + rd_a + (r & 1) * kRowBytes + (r >> 1) * 32);
      else
        f.b[(r - 16) >> 1][r & 1] = tr_read(st + rd_b + (r & 1) * kRowBytes + ((r - 16) >> 1) * 32);
    }
  };
  // products m0 .. m1 - 1 of the 32 (column block j = m / 8, row block i = m % 8)
  auto mma = [&](const Frag& f, int m0, int m1) {
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      if (m < m0 || m >= m1) continue;
      const int j = m >> 3, i = m & 7;
      acc[i][j] = mfma_tr(f.a[i][0], f.a[i][1], f.b[j][0], f.b[j][1], acc[i][j]);
    }
  };

  unsigned char* L0 = g_lds0;
  unsigned char* L1 = g_lds1;
  unsigned char* L2 = g_lds2;
  unsigned char* L3 = g_lds3;
  Frag F0, F1;

  // Prologue: stages 0..2 in flight; once stage 0 has landed everywhere, its
  // operands go to registers and stage 3 fills the fourth slot.
  if (nstage > 0) issue(L0);
  if (nstage > 1) issue(L1);
  if (nstage > 2) issue(L2);
  if (nstage > 2)
    wait_vm<8>();
  else if (nstage > 1)
    wait_vm<4>();
  else
    wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  if (nstage > 0) read_frags(L0, F0, 0, 24);
  if (nstage > 3) issue(L3);

  // Step s (stage s's operands are in `cur`): wait for this wave's loads of
  // stage s+1 (those of s+2 and s+3 may stay in flight) and for its LDS reads
  // of stage s; the barrier then certifies that stage s+1 has landed for every
  // wave and that no wave still reads stage s's slot, which is refilled with
  // stage s+4; stage s+1's operands are read while stage s's products run.
  auto step = [&](int s, const Frag& cur, Frag& next, const unsigned char* next_lds,
                  unsigned char* refill) {
    const int ahead = nstage - 2 - s;  // stages issued beyond s+1
    if (ahead >= 2)
      wait_vm<8>();
    else if (ahead == 1)
      wait_vm<4>();
    else
      wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    // Unconditional, so that the reads and the products share one basic block
    // and can be interleaved: after the last stage this reads a slot that no
    // later stage fills, and those operands are never used.  The first eight
    // products go ahead of the refill's DMA, so that the matrix pipe restarts
    // right after the barrier.
    read_frags(next_lds, next, 0, 8);
    mma(cur, 0, 8);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    if (s + 4 < nstage) issue(refill);
    read_frags(next_lds, next, 8, 24);
    mma(cur, 8, 32);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // The visiting order's sample of the stage group starting at stage s: the
  // group never straddles two samples (T % 128 == 0), so the sample changes
  // exactly at next_bd, every T / 32 stages after the first change (kept as a
  // counter: a 64-bit division per group cost as much as the group's barrier).
  float cur_c = 1.f;
  int64_t cur_seg = -1;
  int next_bd = 0;
  if (MODE == 0 && nstage > 0) {
    cur_seg = kv0 / T;
    cur_c = cvec[order[cur_seg]];
    next_bd = static_cast<int>(((cur_seg + 1) * T - kv0) / kGK);
  }
  for (int s = 0; s < nstage; s += kNStage) {
    if (MODE == 0 && s == next_bd) {
      ++cur_seg;
      next_bd += T / kGK;
      const float c_new = cvec[order[cur_seg]];
      const float ratio = cur_c / c_new;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] *= ratio;
      cur_c = c_new;
    }
    step(s, F0, F1, L1, L0);
    if (s + 1 < nstage) step(s + 1, F1, F0, L2, L1);
    if (s + 2 < nstage) step(s + 2, F0, F1, L3, L2);
    if (s + 3 < nstage) step(s + 3, F1, F0, L0, L3);
  }
  const float fin = (MODE == 0 && cur_seg >= 0) ? cur_c : 1.f;

  // Epilogue: lane (n = lane % 16, g) holds rows 4 g + r of column n of each block.
  float* dst = out + static_cast<int64_t>(z) * p * d;
  float* tile = dst + static_cast<int64_t>(o0 + wm * 128) * d + q0 + wn * 64;
  const uint32_t lane_off = static_cast<uint32_t>((4 * g * d + li) * 4);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      unsigned char* rowp =
          reinterpret_cast<unsigned char*>(tile + static_cast<int64_t>(i * 16 + r) * d);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float*>(rowp + lane_off + j * 64) = acc[i][j][r] * fin;
    }
}

template <int MODE>
__global__ void __launch_bounds__(512, 1) k_gemm_tokens(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ G, int T, int d, int p,
    const float* __restrict__ cvec, const int* __restrict__ order, const int* __restrict__ count,
    int64_t split_tokens, float* __restrict__ out) {
  int ot, qt, z;
  tile_of(blockIdx.x, p / kGM, d / kGN, gridDim.x, ot, qt, z);
  gemm_tile<MODE>(A, G, T, d, p, cvec, order, count, split_tokens, ot, qt, z, out);
}

// The clipped sums of several layers in one launch: the flattened tile list is
// layer 0's tiles, then layer 1's, ..., repeated once per token split; the
// workgroup -> tile mapping deals contiguous runs of it to the XCDs as above,
// so that an XCD works on one or two layers at a time.
__global__ void __launch_bounds__(512, 1) k_gemm_tokens_layers(
    int T, const float* __restrict__ cvec, const int* __restrict__ order,
    const int* __restrict__ count, int64_t split_tokens, GemmLayers tab) {
  const int l = xcd_dealt(blockIdx.x, gridDim.x);
  const int tiles = tab.tile0[tab.n];
  const int z = l / tiles;
  int t = l - z * tiles;
  int i = 0;
  while (i + 1 < tab.n && t >= tab.tile0[i + 1]) ++i;
  t -= tab.tile0[i];
  const int d = tab.d[i], p = tab.p[i];
  int ot, qt;
  tile_in_grid(t, p / kGM, d / kGN, ot, qt);
  gemm_tile<0>(tab.A[i], tab.G[i], T, d, p, cvec, order, count, split_tokens, ot, qt, z,
               tab.out[i]);
}

bool mfma_gemm_ok(int T, int d, int p) {
  return T > 0 && T % kGroup == 0 && d % kGN == 0 && p % kGM == 0;
}

// Split the token range so that there are about 256 workgroups; each split is
// a whole number of 128-token groups.
int mfma_gemm_splits(int B, int T, int d, int p) {
  return mfma_gemm_splits_tiles(B, T, static_cast<int64_t>(p / kGM) * (d / kGN));
}

int mfma_gemm_splits_tiles(int B, int T, int64_t tiles) {
  int64_t want = (256 + tiles - 1) / (tiles > 0 ? tiles : 1);
  const int64_t groups = static_cast<int64_t>(B) * T / kGroup;
  if (want > groups) want = groups;
  if (want < 1) want = 1;
  return static_cast<int>(want);
}

hipError_t launch_aggregate_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p,
                                 const float* c, const int* order, const int* count, int nsplit,
                                 float* part, hipStream_t s) {
  if (!mfma_gemm_ok(T, d, p) || nsplit < 1) return hipErrorInvalidValue;
  const int64_t total = static_cast<int64_t>(B) * T;
  int64_t per = (total + nsplit - 1) / nsplit;
  per = (per + kGroup - 1) / kGroup * kGroup;
  hipLaunchKernelGGL(k_gemm_tokens<0>, dim3((p / kGM) * (d / kGN) * nsplit), dim3(64 * kWaves), 0, s,
                     A, G, T, d, p, c, order, count, per, part);
  return hipGetLastError();
}

int mfma_gemm_tiles(int d, int p) { return (p / kGM) * (d / kGN); }

hipError_t launch_aggregate_mfma_layers(int B, int T, const GemmLayers& tab, const float* c,
                                        const int* order, const int* count, int nsplit,
                                        hipStream_t s) {
  if (tab.n < 1 || tab.n > kGemmLayersMax || nsplit < 1) return hipErrorInvalidValue;
  int tiles = 0;
  for (int i = 0; i < tab.n; ++i) {
    if (!mfma_gemm_ok(T, tab.d[i], tab.p[i]) || tab.tile0[i] != tiles) return hipErrorInvalidValue;
    tiles += mfma_gemm_tiles(tab.d[i], tab.p[i]);
  }
  if (tab.tile0[tab.n] != tiles) return hipErrorInvalidValue;
  const int64_t total = static_cast<int64_t>(B) * T;
  int64_t per = (total + nsplit - 1) / nsplit;
  per = (per + kGroup - 1) / kGroup * kGroup;
  hipLaunchKernelGGL(k_gemm_tokens_layers, dim3(tiles * nsplit), dim3(64 * kWaves), 0, s, T, c,
                     order, count, per, tab);
  return hipGetLastError();
}

hipError_t launch_fgc_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p, float* M,
                           hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (!mfma_gemm_ok(T, d, p)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gemm_tokens<1>, dim3((p / kGM) * (d / kGN) * B), dim3(64 * kWaves), 0, s, A, G,
                     T, d, p, nullptr, nullptr, nullptr, static_cast<int64_t>(T), M);
  return hipGetLastError();
}

}  // namespace dprc
