// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher enqueues on `s` and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dprc {

typedef uint16_t bf16_t;

// Status bit ORed by the clip kernel when some squared norm is not finite.
#define DPRC_STATUS_NONFINITE 1u

// ---- random streams (rng_kernels.hip) ----
hipError_t launch_philox_u32(uint64_t seed, const uint32_t* ctr, uint32_t* out, size_t n,
                             hipStream_t s);
// Probe P^T of `nsamp` samples (sample index = sample0 + i): out[i][j][r] for
// j < kpad, r < p; columns j >= kfill are zero.
// signs: Rademacher +-1 entries instead of normals (same counters and lanes).
hipError_t launch_probe_fill_f32(uint64_t seed, uint32_t layer, uint32_t sample0, int nsamp,
                                 int p, int kfill, int kpad, float* out, hipStream_t s,
                                 bool signs = false);
// The bf16 fill also clears zero[0 .. nzero) (counters used by a later kernel
// of the same call), saving a launch.
hipError_t launch_probe_fill_bf16(uint64_t seed, uint32_t layer, uint32_t sample0, int nsamp,
                                  int p, int kfill, int kpad, bf16_t* out, hipStream_t s,
                                  bool signs = false);
// Probes of several layers in one launch (bf16, kpad columns): layer t's block
// [nsamp][kpad][p[t]] starts at element off[t] of out; bstart[t] = first
// workgroup of layer t (256 row groups of 4 per workgroup), bstart[n] = total.
constexpr int kProbeLayersMax = 64;
template <int N>
struct ProbeLayerTable {
  int n;
  uint32_t layer[N];
  int p[N];
  int64_t off[N];
  int bstart[N + 1];
};
hipError_t launch_probe_fill_layers_bf16(uint64_t seed, const ProbeLayerTable<kProbeLayersMax>& tab,
                                         int nsamp, int kfill, int kpad, bf16_t* out,
                                         hipStream_t s, bool signs);
hipError_t launch_noise_fill(uint64_t seed, uint32_t layer, uint64_t offset, size_t n, float* xi,
                             hipStream_t s);
hipError_t launch_noise_update(float* theta, const float* S, int64_t n, float sigmaC,
                               float eta_over_B, uint64_t seed, uint32_t layer, hipStream_t s);
// The same update reading the clipped sum as nsplit fp32 planes part[split][e]
// (summed in split order, bit-identical to a separate reduction); the sum is
// also stored to S_out unless it is null.
hipError_t launch_noise_update_splits(float* theta, const float* part, int nsplit, int64_t n,
                                      float* S_out, float sigmaC, float eta_over_B, uint64_t seed,
                                      uint32_t layer, hipStream_t s);

// ---- generic VALU kernels, any shape, fp32 math (generic_kernels.hip) ----
// Y[b][j][t] = sum_r X[b][t][r] * P[b or 0][j][r]; P fp32 [.][kp][W].
template <typename TIn>
hipError_t launch_sketch_generic(const TIn* X, int B, int T, int W, const float* P,
                                 int64_t p_bstride, int kp, float* Y, hipStream_t s);
// Z[b][j][q] = sum_t X[b][t][q] * Y[b][j][t].
template <typename TIn>
hipError_t launch_project_generic(const TIn* X, int B, int T, int W, const float* Y, int kp,
                                  float* Z, hipStream_t s);
// part[b][chunk] = sum over (j, q) of w_j (sum_split Z[b][split][j][q])^2, with
// w_j = w0 for j < n0, w1 for n0 <= j < n0 + n1, 0 otherwise.
hipError_t launch_frob_partial(const float* Z, int B, int nsplit, int kp, int W, int n0, float w0,
                               int n1, float w1, double* part, int nchunk, hipStream_t s);
// n[b] = (accumulate ? n[b] : 0) + sum_c part[b][c].
hipError_t launch_sum_parts(const double* part, int B, int nparts, float* n, int accumulate,
                            hipStream_t s);
// Z[b][j][q] = sum_split Zp[b][split][j][q] (fp32) and optionally a bf16 copy.
hipError_t launch_sum_splits(const float* Zp, int B, int nsplit, int rows, int W, float* Z,
                             bf16_t* Zb, hipStream_t s);
template <typename TIn>
hipError_t launch_ghost_generic(const TIn* A, const TIn* G, int B, int T, int d, int p,
                                double* part, int* nparts_out, hipStream_t s);
int ghost_generic_nparts(int T);
template <typename TIn>
hipError_t launch_fgc_generic(const TIn* A, const TIn* G, int B, int T, int d, int p, float* M,
                              hipStream_t s);
template <typename TIn>
hipError_t launch_aggregate_generic(const TIn* A, const TIn* G, int B, int T, int d, int p,
                                    const float* c, float* S, hipStream_t s);
// c[i], optional c_out, status bit, and the active samples in ascending c order.
hipError_t launch_clip(const float* n, int B, float C, float* c, float* c_out, uint32_t* status,
                       int* order, int* count, hipStream_t s);
// w[1] = w[0], w[0] = 0 (one atomic exchange).
// out[x] (x < nblocks) = XOR of the 16-byte words workgroup x read of in[0 .. n16).
hipError_t launch_stream_read(const void* in, int64_t n16, uint32_t* out, int nblocks,
                              hipStream_t s);
hipError_t launch_take_status(uint32_t* w, hipStream_t s);
// out[e] = sum_{sp < nsplit} part[sp][e].
hipError_t launch_reduce_splits(const float* part, int nsplit, int64_t n, float* out, hipStream_t s);
// Hutch++ probe for the last pass: rows 0..s-1 = orthonormal basis of the s
// sketch rows (CholeskyQR2), rows s..s+r-1 = W - Q Q^T W.  The sketch is the
// sum over nsplit partials: X[b][i][e] = sum_sp Xp[b * x_bstride + sp *
// split_stride + i * p + e].  W rows t < r at W[b * w_bstride + t * p].
// P3 fp32 [B][s+r][p] holds the first-pass basis and, when P3b is null, the
// result; otherwise the result goes to P3b bf16 [B][p3b_rows][p] with zero
// rows from s+r on.  `scratch`: hpp_orth_scratch_bytes() of device memory.
hipError_t launch_hpp_orth(const float* Xp, int nsplit, int64_t split_stride, int64_t x_bstride,
                           const float* W, int64_t w_bstride, int B, int p, int s, int r,
                           float* P3, bf16_t* P3b, int p3b_rows, double* scratch, hipStream_t st);
size_t hpp_orth_scratch_bytes(int B, int p, int s, int r);

// Poisson subsampling: idx[0, min(|B|, cap)) = ascending indices n < N whose
// membership word is below thr; *count = |B| (device).  counts: workspace of
// poisson_blocks(N) int64.
int64_t poisson_blocks(int64_t N);
hipError_t launch_poisson_sample(uint64_t seed, uint32_t step, int64_t N, uint64_t thr,
                                 int64_t* idx, int64_t cap, int64_t* count, int64_t* counts,
                                 hipStream_t s);

// ---- parameters that are not linear layers (other_layers.hip) ----
// RMSNorm gain: part [B][nsplit][d] fp32 scratch; v [B][d] (may be null);
// n_sq[b] (= or +=) ||v_b||^2.
// sq [B][rmsnorm_sq_chunks(d)] fp64 scratch.
int rmsnorm_splits(int B, int T, int d);
int rmsnorm_sq_chunks(int d);
template <typename TIn>
hipError_t launch_rmsnorm_norm(const TIn* X, const TIn* D, int B, int T, int d, float* part,
                               int nsplit, double* sq, float* v, float* n_sq, int accumulate,
                               hipStream_t s);
// S[c] = sum_i c_i v[i][c].
hipError_t launch_weighted_rows(const float* v, const float* c, int B, int d, float* S,
                                hipStream_t s);

// Embedding table: per-sample sort of (id, position) (1 <= T <= 16384); the
// segmented sums over splits of the sorted positions (pieces of the groups
// that cross splits in head/tail [B][nsplit][d], joined in split order); the
// table update through a per-sample row map [B][V] and group sums [B][T][d].
int emb_splits(int B, int T, int d);
int emb_combine_chunks(int d);
hipError_t launch_emb_sort(const int32_t* ids, int B, int T, int32_t* spos, int32_t* sid,
                           int32_t* gidp, int32_t* ustart, int32_t* uid, int32_t* ng,
                           hipStream_t s);
// part [B][nsplit][ceil(d / 2048)] and cpart [B][emb_combine_chunks(d)] fp64.
template <typename TIn>
hipError_t launch_emb_norm(const TIn* D, int B, int T, int d, const int32_t* spos,
                           const int32_t* sid, const int32_t* gidp, int nsplit, double* part,
                           float* head, float* tail, double* cpart, float* n_sq, int accumulate,
                           hipStream_t s);
template <typename TIn>
hipError_t launch_emb_group_sums(const TIn* D, int B, int T, int d, const int32_t* spos,
                                 const int32_t* sid, const int32_t* gidp, int nsplit, float* head,
                                 float* tail, float* gsum, hipStream_t s);
hipError_t launch_emb_update(const float* gsum, int B, int T, int d, const int32_t* uid,
                             const int32_t* ng, int32_t* rowmap, int V, const float* c, float* E,
                             float sigmaC, float eta_over_B, uint64_t seed, uint32_t layer,
                             hipStream_t s);
hipError_t launch_emb_zero_norm(int B, float* n_sq, int accumulate, hipStream_t s);

// ---- MFMA kernels for bf16 inputs (mfma_hutch.hip, mfma_gemm.hip) ----
constexpr int kMfmaProbeCols = 32;  // padded probe width of the MFMA Hutch path
bool mfma_sketch_ok(int T, int W);
// Several layers per launch of the Hutch passes (layer tables in the kernel
// arguments, kNormLayersMax per launch).
constexpr int kNormLayersMax = 40;
struct SketchLayers {
  int n;
  const bf16_t* X[kNormLayersMax];
  const bf16_t* P[kNormLayersMax];
  bf16_t* Y[kNormLayersMax];
  int W[kNormLayersMax];
  int64_t pbs[kNormLayersMax];
};
struct ProjectLayers {
  int n;
  const bf16_t* X[kNormLayersMax];
  const bf16_t* Y[kNormLayersMax];
  int W[kNormLayersMax];
  int64_t pbase[kNormLayersMax];
};
// 2: 128-token workgroups of 8 waves, 1: 64 tokens, 4 waves, 0: 32 tokens, 4 waves.
int mfma_sketch_variant(int B, int T, int W);
// The sketch of every layer of the table (all of shape class `variant`).
hipError_t launch_sketch_mfma_layers(int variant, int B, int T, const SketchLayers& tab,
                                     hipStream_t s);
// The fused projection-and-square of every layer of the table (all with column
// block `cols`); layer l's partials at part + pbase[l], row stride part_stride.
hipError_t launch_project_sq_mfma_layers(int B, int T, int cols, const ProjectLayers& tab, int n0,
                                         float w0, int n1, float w1, double* part,
                                         int64_t part_stride, hipStream_t s);
bool mfma_project_ok(int T, int W);
int mfma_project_splits(int B, int T, int W);
// Y[b][j][t] (bf16, [B][32][T]) = sum_r X[b][t][r] P[b or 0][j][r], P bf16 [.][32][W].
hipError_t launch_sketch_mfma(const bf16_t* X, int B, int T, int W, const bf16_t* P,
                              int64_t p_bstride, bf16_t* Y, hipStream_t s);
// Zp[b][split][j][q] (fp32, j < 32) = sum_{t in split} X[b][t][q] Y[b][j][t].
hipError_t launch_project_mfma(const bf16_t* X, int B, int T, int W, const bf16_t* Y, int nsplit,
                               float* Zp, hipStream_t s);
// Column block (128 or 64) of the fused projection-and-square, 0 if it would
// give fewer than 256 workgroups.
int mfma_project_sq_cols(int B, int T, int W);
// part[b * part_stride + blk] (fp64, blk < W / cols) = sum_j w_j sum_{q in block}
// (sum_t X[b][t][q] Y[b][j][t])^2, w_j as in launch_frob_finish; whole token
// range in one workgroup per block.
hipError_t launch_project_sq_mfma(const bf16_t* X, int B, int T, int W, const bf16_t* Y, int cols,
                                  int n0, float w0, int n1, float w1, double* part,
                                  int64_t part_stride, hipStream_t s);
// n_sq[b] (= or +=) sum_j w_j ||sum_split Zp[b][split][j][:]||^2 with w_j = w0
// for j < n0, w1 for n0 <= j < n0 + n1, else 0 (W % 4 == 0).  Fixed-order fp64
// sums through part [B][mfma_frob_chunks(W)] (workspace), then k_sum_parts.
int mfma_frob_chunks(int W);
hipError_t launch_frob_finish(const float* Zp, int B, int nsplit, int W, int n0, float w0, int n1,
                              float w1, double* part, float* n_sq, int accumulate, hipStream_t s);

// Ghost norm per sample from 128 x 128 Gram tile pairs: part[b][pair] (fp64).
bool mfma_ghost_ok(int T, int d, int p);
int mfma_ghost_nparts(int T);
hipError_t launch_ghost_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p,
                             double* part, hipStream_t s);

bool mfma_gemm_ok(int T, int d, int p);
int mfma_gemm_splits(int B, int T, int d, int p);
// Token splits for `tiles` 256 x 256 output tiles: about 256 workgroups.
int mfma_gemm_splits_tiles(int B, int T, int64_t tiles);
// 256 x 256 output tiles of a p x d clipped sum.
int mfma_gemm_tiles(int d, int p);
// Several layers' clipped sums in one launch (layer table in the kernel
// arguments): layer i owns the flattened tiles tile0[i] .. tile0[i + 1] - 1,
// tile0[0] = 0, and its token-split planes out[i][split][o][q].
constexpr int kGemmLayersMax = 16;
struct GemmLayers {
  int n;
  int tile0[kGemmLayersMax + 1];
  int d[kGemmLayersMax];
  int p[kGemmLayersMax];
  const bf16_t* A[kGemmLayersMax];
  const bf16_t* G[kGemmLayersMax];
  float* out[kGemmLayersMax];
};
hipError_t launch_aggregate_mfma_layers(int B, int T, const GemmLayers& tab, const float* c,
                                        const int* order, const int* count, int nsplit,
                                        hipStream_t s);
// Clipped sum over the active samples order[0..*count) (ascending c):
// part[split][o][q] = sum over the split's tokens of c G[t][o] A[t][q].
hipError_t launch_aggregate_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p,
                                 const float* c, const int* order, const int* count, int nsplit,
                                 float* part, hipStream_t s);
// Per-sample materialised gradients M[b][o][q] = sum_t G_b[t][o] A_b[t][q] (FGC).
hipError_t launch_fgc_mfma(const bf16_t* A, const bf16_t* G, int B, int T, int d, int p, float* M,
                           hipStream_t s);

// ---- MLP block forward / backward pass 1 (block_kernels.hip) ----
bool gemm_nt_ok(int64_t M, int N, int K1, int K2, int K3);
hipError_t launch_gemm_nt(const bf16_t* A1, const bf16_t* B1, int K1, const bf16_t* A2,
                          const bf16_t* B2, int K2, int64_t M, int N, const bf16_t* Rz, bf16_t* C,
                          hipStream_t s);
// The same over three (A, B) pairs (K3 > 0 needs K2 > 0).
hipError_t launch_gemm_nt3(const bf16_t* A1, const bf16_t* B1, int K1, const bf16_t* A2,
                           const bf16_t* B2, int K2, const bf16_t* A3, const bf16_t* B3, int K3,
                           int64_t M, int N, const bf16_t* Rz, bf16_t* C, hipStream_t s);
hipError_t launch_rmsnorm_fwd(const bf16_t* x, const float* gamma, int64_t M, int d, float eps,
                              bf16_t* xhat, bf16_t* y, float* rstd, hipStream_t s);
hipError_t launch_rmsnorm_bwd(const bf16_t* x, const float* rstd, const float* gamma,
                              const bf16_t* dy, const bf16_t* dout, int64_t M, int d, bf16_t* dx,
                              hipStream_t s);
// y [M][d] against Wg, Wu [f][d]: g, u and h = silu(g) u, each [M][f] (f % 128 == 0).
hipError_t launch_gemm_nt_swiglu(const bf16_t* y, const bf16_t* Wg, const bf16_t* Wu, int d,
                                 int64_t M, int f, bf16_t* g, bf16_t* u, bf16_t* h, hipStream_t s);
// dh = dout WdT^T ([M][f], not stored), then dg = dh u silu'(g), du = dh silu(g).
hipError_t launch_gemm_nt_swiglu_bwd(const bf16_t* dout, const bf16_t* WdT, int d, int64_t M, int f,
                                     const bf16_t* g, const bf16_t* u, bf16_t* dg, bf16_t* du,
                                     hipStream_t s);
hipError_t launch_cast_transpose(const float* theta, int p, int d, bf16_t* W, bf16_t* Wt,
                                 hipStream_t s);

// ---- attention block (attn_kernels.hip): head width 64, T % 128 == 0 ----
bool attn_shape_ok(int T, int H, int KV);
// In place RoPE on x [M][nh * 64] (row % T is the position); inverse rotates back.
hipError_t launch_rope(bf16_t* x, int64_t M, int T, int nh, double base, bool inverse,
                       hipStream_t s);
// Causal grouped-query attention: q [B T][H 64], k, v [B T][KV 64] -> o [B T][H 64]
// and lse [B][H][T] (natural log of each softmax row's normaliser).
hipError_t launch_attn_fwd(const bf16_t* q, const bf16_t* k, const bf16_t* v, int B, int T, int H,
                           int KV, bf16_t* o, float* lse, hipStream_t s);
// dq, dk, dv from dO (Dvec: B H T floats of scratch for rowsum(dO o)).
size_t attn_bwd_scratch_bytes(int B, int T, int H);
hipError_t launch_attn_bwd(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* o,
                           const float* lse, const bf16_t* dO, int B, int T, int H, int KV,
                           float* Dvec, bf16_t* dq, bf16_t* dk, bf16_t* dv, hipStream_t s);

}  // namespace dprc
