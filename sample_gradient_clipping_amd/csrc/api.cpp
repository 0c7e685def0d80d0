// C ABI of libdprc (declared in include/dprc.h): host-side validation,
// workspace layout and launch sequencing.  No allocation, no synchronisation,
// no mutable global state; everything is enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "dprc.h"
#include "internal.h"

using namespace dprc;

static_assert(DPRC_STATUS_NONFINITE == DP_STATUS_NONFINITE_NORM, "status bit mismatch");

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kInvalid = static_cast<size_t>(-1);
// Every call that forms clip factors keeps its sticky status word at byte 0 of
// its workspace (read and cleared by dp_read_device_status); the word after it
// receives the value being read.
constexpr size_t kStatusBytes = 8;
constexpr int kMaxDevices = 64;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sequential carve-out of one workspace.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// One frob block per ~1K elements: enough blocks to stream the partials at
// full bandwidth.
int frob_chunks(int64_t elems) {
  int64_t c = elems / 1024;
  if (c < 1) c = 1;
  if (c > 1024) c = 1024;
  return static_cast<int>(c);
}

// ---- dp_norm_est planning ----
struct NormPlan {
  bool mfma = false;
  int s = 0, r = 0, k3 = 0;  // Hutch++ split
  int nsplit_d = 1, nsplit_p = 1, nchunk = 1, nparts = 0;
  int sq_cols = 0;  // MFMA Hutch final pass: fused projection-and-square column block, 0 = split + finish
  // offsets (bytes) into the workspace; unused ones stay 0
  size_t pf = 0, pb = 0, y = 0, yb = 0, z = 0, zp = 0, z1b = 0, v = 0, xp = 0, x = 0, p3 = 0,
         p3b = 0, m = 0, part = 0, orth = 0;
  size_t total = 0;
};

bool valid_method(int m) { return m >= DP_NORM_HUTCH && m <= DP_NORM_FGC; }
bool valid_dtype(int t) { return t == DP_F32 || t == DP_BF16; }

bool norm_args_ok(int method, int dtype, int B, int T, int d, int p, int k) {
  if (!valid_method(method) || !valid_dtype(dtype)) return false;
  if (B < 0 || T < 0 || d < 1 || p < 1) return false;
  if (static_cast<int64_t>(T) * (d > p ? d : p) > (static_cast<int64_t>(1) << 40)) return false;
  if (method == DP_NORM_HUTCH && (k < 1 || k > p)) return false;
  if (method == DP_NORM_HUTCHPP && (k < 3 || k > p || k / 3 > 32 || k - 2 * (k / 3) > 32))
    return false;
  return true;
}

NormPlan plan_norm(int method, int dtype, int B, int T, int d, int p, int k) {
  NormPlan P;
  Carver cv;
  const size_t Bz = static_cast<size_t>(B);
  const size_t f4 = 4, h2 = 2;
  const bool bf = dtype == DP_BF16;
  if (method == DP_NORM_HUTCH) {
    P.mfma = bf && k <= kMfmaProbeCols && mfma_sketch_ok(T, p) && mfma_project_ok(T, d);
    if (P.mfma) {
      P.sq_cols = mfma_project_sq_cols(B, T, d);
      P.pb = cv.take(Bz * kMfmaProbeCols * p * h2);
      P.yb = cv.take(Bz * kMfmaProbeCols * T * h2);
      if (P.sq_cols > 0) {
        P.part = cv.take(Bz * (d / P.sq_cols) * sizeof(double));
      } else {
        P.nsplit_d = mfma_project_splits(B, T, d);
        P.zp = cv.take(Bz * P.nsplit_d * kMfmaProbeCols * d * f4);
        P.part = cv.take(Bz * mfma_frob_chunks(d) * sizeof(double));
      }
    } else {
      P.pf = cv.take(Bz * k * p * f4);
      P.y = cv.take(Bz * k * T * f4);
      P.z = cv.take(Bz * k * d * f4);
      P.nchunk = frob_chunks(static_cast<int64_t>(k) * d);
    }
  } else if (method == DP_NORM_HUTCHPP) {
    P.s = k / 3;
    P.r = k - 2 * P.s;
    P.k3 = P.s + P.r;
    P.mfma = bf && P.k3 <= kMfmaProbeCols && mfma_sketch_ok(T, p) && mfma_sketch_ok(T, d) &&
             mfma_project_ok(T, d) && mfma_project_ok(T, p);
    P.pf = cv.take(Bz * P.k3 * p * f4);
    P.p3 = cv.take(Bz * P.k3 * p * f4);
    P.orth = cv.take(hpp_orth_scratch_bytes(B, p, P.s, P.r));
    if (P.mfma) {
      P.nsplit_d = mfma_project_splits(B, T, d);
      P.nsplit_p = mfma_project_splits(B, T, p);
      P.pb = cv.take(Bz * kMfmaProbeCols * p * h2);
      P.yb = cv.take(Bz * kMfmaProbeCols * T * h2);
      P.zp = cv.take(Bz * P.nsplit_d * kMfmaProbeCols * d * f4);
      P.z1b = cv.take(Bz * kMfmaProbeCols * d * h2);
      P.xp = cv.take(Bz * P.nsplit_p * kMfmaProbeCols * p * f4);
      P.p3b = cv.take(Bz * kMfmaProbeCols * p * h2);
      P.sq_cols = mfma_project_sq_cols(B, T, d);
      P.part = cv.take(Bz * (P.sq_cols > 0 ? d / P.sq_cols : mfma_frob_chunks(d)) * sizeof(double));
    } else {
      P.y = cv.take(Bz * P.k3 * (T > 0 ? T : 1) * f4);
      P.z = cv.take(Bz * P.k3 * d * f4);
      P.v = cv.take(Bz * P.s * (T > 0 ? T : 1) * f4);
      P.x = cv.take(Bz * P.s * p * f4);
      P.nchunk = frob_chunks(static_cast<int64_t>(P.k3) * d);
    }
  } else if (method == DP_NORM_GHOST) {
    P.mfma = bf && mfma_ghost_ok(T, d, p);
    P.nparts = P.mfma ? mfma_ghost_nparts(T) : ghost_generic_nparts(T);
    P.nchunk = P.nparts;
  } else {  // FGC
    P.mfma = bf && mfma_gemm_ok(T, d, p);
    P.m = cv.take(Bz * p * d * f4);
    P.nchunk = frob_chunks(static_cast<int64_t>(p) * d);
  }
  const int nparts = method == DP_NORM_GHOST ? P.nparts : P.nchunk;
  if (!P.mfma || method == DP_NORM_GHOST || method == DP_NORM_FGC)  // MFMA Hutch: taken above
    P.part = cv.take(Bz * (nparts > 0 ? nparts : 1) * sizeof(double));
  P.total = cv.off;
  return P;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + off);
}

// Optional timing events recorded around a call's main kernels (may be null).
struct Marks {
  hipEvent_t begin = nullptr, end = nullptr;
  hipError_t open(hipStream_t s) const { return begin ? hipEventRecord(begin, s) : hipSuccess; }
  hipError_t close(hipStream_t s) const { return end ? hipEventRecord(end, s) : hipSuccess; }
};

#define DP_TRY(expr)                          \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return DP_ERR_HIP;  \
  } while (0)

template <typename TIn>
dp_status_t run_norm_generic_hutch(const NormPlan& P, int B, int T, int d, int p, int k,
                                   const TIn* A, const TIn* G, uint64_t seed, uint32_t layer,
                                   bool shared, bool signs, bool accum, float* n_sq, void* ws, hipStream_t s,
                                   const Marks& mk) {
  float* Pf = at<float>(ws, P.pf);
  float* Y = at<float>(ws, P.y);
  float* Z = at<float>(ws, P.z);
  double* part = at<double>(ws, P.part);
  const int nS = shared ? 1 : B;
  const int64_t pbs = shared ? 0 : static_cast<int64_t>(k) * p;
  DP_TRY(launch_probe_fill_f32(seed, layer, 0, nS, p, k, k, Pf, s, signs));
  DP_TRY(mk.open(s));
  DP_TRY(launch_sketch_generic<TIn>(G, B, T, p, Pf, pbs, k, Y, s));
  DP_TRY(launch_project_generic<TIn>(A, B, T, d, Y, k, Z, s));
  DP_TRY(mk.close(s));
  DP_TRY(launch_frob_partial(Z, B, 1, k, d, k, 1.0f / k, 0, 0.f, part, P.nchunk, s));
  DP_TRY(launch_sum_parts(part, B, P.nchunk, n_sq, accum ? 1 : 0, s));
  return DP_OK;
}

dp_status_t run_norm_mfma_hutch(const NormPlan& P, int B, int T, int d, int p, int k,
                                const bf16_t* A, const bf16_t* G, uint64_t seed, uint32_t layer,
                                bool shared, bool signs, bool accum, float* n_sq, void* ws, hipStream_t s,
                                const Marks& mk) {
  bf16_t* Pb = at<bf16_t>(ws, P.pb);
  bf16_t* Yb = at<bf16_t>(ws, P.yb);
  float* Zp = at<float>(ws, P.zp);
  const int nS = shared ? 1 : B;
  const int64_t pbs = shared ? 0 : static_cast<int64_t>(kMfmaProbeCols) * p;
  DP_TRY(launch_probe_fill_bf16(seed, layer, 0, nS, p, k, kMfmaProbeCols, Pb, s, signs));
  DP_TRY(mk.open(s));
  DP_TRY(launch_sketch_mfma(G, B, T, p, Pb, pbs, Yb, s));
  if (P.sq_cols > 0) {
    double* part = at<double>(ws, P.part);
    DP_TRY(launch_project_sq_mfma(A, B, T, d, Yb, P.sq_cols, k, 1.0f / k, 0, 0.f, part, d / P.sq_cols, s));
    DP_TRY(mk.close(s));
    DP_TRY(launch_sum_parts(part, B, d / P.sq_cols, n_sq, accum ? 1 : 0, s));
    return DP_OK;
  }
  DP_TRY(launch_project_mfma(A, B, T, d, Yb, P.nsplit_d, Zp, s));
  DP_TRY(mk.close(s));
  DP_TRY(launch_frob_finish(Zp, B, P.nsplit_d, d, k, 1.0f / k, 0, 0.f, at<double>(ws, P.part), n_sq,
                            accum ? 1 : 0, s));
  return DP_OK;
}

template <typename TIn>
dp_status_t run_norm_generic_hpp(const NormPlan& P, int B, int T, int d, int p, const TIn* A,
                                 const TIn* G, uint64_t seed, uint32_t layer, bool shared,
                                 bool signs, bool accum, float* n_sq, void* ws, hipStream_t s,
                                 const Marks& mk) {
  const int S_ = P.s, R_ = P.r, K3 = P.k3;
  float* Pf = at<float>(ws, P.pf);
  float* P3 = at<float>(ws, P.p3);
  float* Y = at<float>(ws, P.y);
  float* Z = at<float>(ws, P.z);
  float* V = at<float>(ws, P.v);
  float* X = at<float>(ws, P.x);
  double* part = at<double>(ws, P.part);
  const int nS = shared ? 1 : B;
  const int64_t pbs = shared ? 0 : static_cast<int64_t>(K3) * p;
  DP_TRY(launch_probe_fill_f32(seed, layer, 0, nS, p, K3, K3, Pf, s, signs));
  // pass 1: Z1 = A^T (G S)
  DP_TRY(mk.open(s));
  DP_TRY(launch_sketch_generic<TIn>(G, B, T, p, Pf, pbs, S_, Y, s));
  DP_TRY(launch_project_generic<TIn>(A, B, T, d, Y, S_, Z, s));
  // pass 2: X = G^T (A Z1) = O S
  DP_TRY(launch_sketch_generic<TIn>(A, B, T, d, Z, static_cast<int64_t>(S_) * d, S_, V, s));
  DP_TRY(launch_project_generic<TIn>(G, B, T, p, V, S_, X, s));
  // Q = orth(X), W' = (I - Q Q^T) W
  DP_TRY(launch_hpp_orth(X, 1, 0, static_cast<int64_t>(S_) * p, Pf + static_cast<int64_t>(S_) * p,
                         pbs, B, p, S_, R_, P3, nullptr, 0, at<double>(ws, P.orth), s));
  // pass 3: head + tail / r
  DP_TRY(launch_sketch_generic<TIn>(G, B, T, p, P3, static_cast<int64_t>(K3) * p, K3, Y, s));
  DP_TRY(launch_project_generic<TIn>(A, B, T, d, Y, K3, Z, s));
  DP_TRY(mk.close(s));
  DP_TRY(launch_frob_partial(Z, B, 1, K3, d, S_, 1.0f, R_, 1.0f / R_, part, P.nchunk, s));
  DP_TRY(launch_sum_parts(part, B, P.nchunk, n_sq, accum ? 1 : 0, s));
  return DP_OK;
}

dp_status_t run_norm_mfma_hpp(const NormPlan& P, int B, int T, int d, int p, const bf16_t* A,
                              const bf16_t* G, uint64_t seed, uint32_t layer, bool shared,
                              bool signs, bool accum, float* n_sq, void* ws, hipStream_t s, const Marks& mk) {
  const int S_ = P.s, R_ = P.r, K3 = P.k3;
  float* Pf = at<float>(ws, P.pf);
  float* P3 = at<float>(ws, P.p3);
  bf16_t* Pb = at<bf16_t>(ws, P.pb);
  bf16_t* Yb = at<bf16_t>(ws, P.yb);
  float* Zp = at<float>(ws, P.zp);
  bf16_t* Z1b = at<bf16_t>(ws, P.z1b);
  float* Xp = at<float>(ws, P.xp);
  bf16_t* P3b = at<bf16_t>(ws, P.p3b);
  const int nS = shared ? 1 : B;
  const int64_t pfs = shared ? 0 : static_cast<int64_t>(K3) * p;
  const int64_t pbs = shared ? 0 : static_cast<int64_t>(kMfmaProbeCols) * p;
  const int64_t pad_d = static_cast<int64_t>(kMfmaProbeCols) * d;
  const int64_t pad_p = static_cast<int64_t>(kMfmaProbeCols) * p;
  DP_TRY(launch_probe_fill_f32(seed, layer, 0, nS, p, K3, K3, Pf, s, signs));
  DP_TRY(launch_probe_fill_bf16(seed, layer, 0, nS, p, S_, kMfmaProbeCols, Pb, s, signs));
  // pass 1: Z1 = A^T (G S)
  DP_TRY(mk.open(s));
  DP_TRY(launch_sketch_mfma(G, B, T, p, Pb, pbs, Yb, s));
  DP_TRY(launch_project_mfma(A, B, T, d, Yb, P.nsplit_d, Zp, s));
  DP_TRY(launch_sum_splits(Zp, B, P.nsplit_d, kMfmaProbeCols, d, nullptr, Z1b, s));
  // pass 2: X = G^T (A Z1)
  DP_TRY(launch_sketch_mfma(A, B, T, d, Z1b, pad_d, Yb, s));
  DP_TRY(launch_project_mfma(G, B, T, p, Yb, P.nsplit_p, Xp, s));
  // Q = orth(X) over the projection's split partials, W' = (I - Q Q^T) W, as bf16 rows
  DP_TRY(launch_hpp_orth(Xp, P.nsplit_p, pad_p, P.nsplit_p * pad_p, Pf + static_cast<int64_t>(S_) * p,
                         pfs, B, p, S_, R_, P3, P3b, kMfmaProbeCols, at<double>(ws, P.orth), s));
  // pass 3
  DP_TRY(launch_sketch_mfma(G, B, T, p, P3b, pad_p, Yb, s));
  if (P.sq_cols > 0) {
    double* part = at<double>(ws, P.part);
    DP_TRY(launch_project_sq_mfma(A, B, T, d, Yb, P.sq_cols, S_, 1.0f, R_, 1.0f / R_, part, d / P.sq_cols, s));
    DP_TRY(mk.close(s));
    DP_TRY(launch_sum_parts(part, B, d / P.sq_cols, n_sq, accum ? 1 : 0, s));
    return DP_OK;
  }
  DP_TRY(launch_project_mfma(A, B, T, d, Yb, P.nsplit_d, Zp, s));
  DP_TRY(mk.close(s));
  DP_TRY(launch_frob_finish(Zp, B, P.nsplit_d, d, S_, 1.0f, R_, 1.0f / R_, at<double>(ws, P.part),
                            n_sq, accum ? 1 : 0, s));
  return DP_OK;
}

template <typename TIn>
dp_status_t run_norm_exact(int method, const NormPlan& P, int B, int T, int d, int p,
                           const TIn* A, const TIn* G, bool accum, float* n_sq, void* ws,
                           hipStream_t s, const Marks& mk) {
  double* part = at<double>(ws, P.part);
  if (method == DP_NORM_GHOST) {
    int np = 0;
    DP_TRY(mk.open(s));
    if constexpr (sizeof(TIn) == 2) {
      if (P.mfma) {
        np = P.nparts;
        DP_TRY(launch_ghost_mfma(A, G, B, T, d, p, part, s));
      } else {
        DP_TRY(launch_ghost_generic<TIn>(A, G, B, T, d, p, part, &np, s));
      }
    } else {
      DP_TRY(launch_ghost_generic<TIn>(A, G, B, T, d, p, part, &np, s));
    }
    DP_TRY(mk.close(s));
    DP_TRY(launch_sum_parts(part, B, np, n_sq, accum ? 1 : 0, s));
    return DP_OK;
  }
  float* M = at<float>(ws, P.m);
  DP_TRY(mk.open(s));
  if constexpr (sizeof(TIn) == 2) {
    if (P.mfma) {
      DP_TRY(launch_fgc_mfma(A, G, B, T, d, p, M, s));
    } else {
      DP_TRY(launch_fgc_generic<TIn>(A, G, B, T, d, p, M, s));
    }
  } else {
    DP_TRY(launch_fgc_generic<TIn>(A, G, B, T, d, p, M, s));
  }
  DP_TRY(mk.close(s));
  DP_TRY(launch_frob_partial(M, B, 1, p, d, p, 1.0f, 0, 0.f, part, P.nchunk, s));
  DP_TRY(launch_sum_parts(part, B, P.nchunk, n_sq, accum ? 1 : 0, s));
  return DP_OK;
}

// ---- dp_clip_aggregate planning ----
struct AggPlan {
  bool mfma = false;
  int nsplit = 1;
  size_t status = 0, c = 0, order = 0, count = 0, part = 0, sbuf = 0, total = 0;
};

// with_sbuf: also a [p][d] buffer for the clipped sum when the caller of the
// fused update passes no S.
// The workspace prefix every clipped-sum plan starts with (it depends on B only).
void carve_agg_prefix(Carver& cv, AggPlan& P, int B) {
  const size_t Bz = static_cast<size_t>(B > 0 ? B : 1);
  P.status = cv.take(kStatusBytes);
  P.c = cv.take(Bz * 4);
  P.order = cv.take(Bz * 4);
  P.count = cv.take(4);
}

AggPlan plan_agg(int dtype, int B, int T, int d, int p, bool with_sbuf = false) {
  AggPlan P;
  Carver cv;
  carve_agg_prefix(cv, P, B);
  P.mfma = dtype == DP_BF16 && B > 0 && mfma_gemm_ok(T, d, p);
  if (P.mfma) {
    P.nsplit = mfma_gemm_splits(B, T, d, p);
    if (P.nsplit > 1) P.part = cv.take(static_cast<size_t>(P.nsplit) * p * d * 4);
  }
  if (with_sbuf) P.sbuf = cv.take(static_cast<size_t>(p) * d * 4);
  P.total = cv.off;
  return P;
}

bool agg_args_ok(int dtype, int B, int T, int d, int p) {
  return valid_dtype(dtype) && B >= 0 && T >= 0 && d >= 1 && p >= 1 &&
         static_cast<int64_t>(T) * (d > p ? d : p) <= (static_cast<int64_t>(1) << 40);
}

}  // namespace

extern "C" {

int dp_abi_version(void) { return DPRC_ABI_VERSION; }

const char* dp_status_string(dp_status_t s) {
  switch (s) {
    case DP_OK: return "DP_OK";
    case DP_ERR_INVALID_ARG: return "DP_ERR_INVALID_ARG: invalid size, pointer, alignment or parameter";
    case DP_ERR_UNSUPPORTED: return "DP_ERR_UNSUPPORTED: combination not implemented";
    case DP_ERR_WORKSPACE: return "DP_ERR_WORKSPACE: workspace smaller than the query";
    case DP_ERR_HIP: return "DP_ERR_HIP: a HIP launch failed";
  }
  return "unknown dp_status_t";
}

size_t dp_norm_est_workspace(int method, int dtype, int B, int T, int d, int p, int k) {
  if (!norm_args_ok(method, dtype, B, T, d, p, k)) return kInvalid;
  return plan_norm(method, dtype, B, T, d, p, k).total;
}

static dp_status_t norm_est_impl(int method, int dtype, int B, int T, int d, int p, int k,
                                 const void* A, const void* G, uint64_t seed, uint32_t layer,
                                 uint32_t flags, float* n_sq, void* ws, size_t ws_bytes,
                                 dp_stream_t stream, const Marks& mk) {
  if (!norm_args_ok(method, dtype, B, T, d, p, k)) return DP_ERR_INVALID_ARG;
  if ((flags & ~(DP_ACCUMULATE | DP_PROBE_SHARED | DP_PROBE_RADEMACHER)) != 0)
    return DP_ERR_INVALID_ARG;
  if (B == 0) return DP_OK;
  if (n_sq == nullptr || !aligned(n_sq, 4)) return DP_ERR_INVALID_ARG;
  if (T > 0 && (A == nullptr || G == nullptr || !aligned(A, 16) || !aligned(G, 16)))
    return DP_ERR_INVALID_ARG;
  const NormPlan P = plan_norm(method, dtype, B, T, d, p, k);
  if (ws_bytes < P.total) return DP_ERR_WORKSPACE;
  if (P.total > 0 && (ws == nullptr || !aligned(ws, 16))) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool accum = (flags & DP_ACCUMULATE) != 0;
  const bool shared = (flags & DP_PROBE_SHARED) != 0;
  const bool signs = (flags & DP_PROBE_RADEMACHER) != 0;
  const bool bf = dtype == DP_BF16;
  const bf16_t* Ab = static_cast<const bf16_t*>(A);
  const bf16_t* Gb = static_cast<const bf16_t*>(G);
  const float* Af = static_cast<const float*>(A);
  const float* Gf = static_cast<const float*>(G);
  switch (method) {
    case DP_NORM_HUTCH:
      if (P.mfma) return run_norm_mfma_hutch(P, B, T, d, p, k, Ab, Gb, seed, layer, shared, signs, accum, n_sq, ws, s, mk);
      return bf ? run_norm_generic_hutch<bf16_t>(P, B, T, d, p, k, Ab, Gb, seed, layer, shared, signs, accum, n_sq, ws, s, mk)
                : run_norm_generic_hutch<float>(P, B, T, d, p, k, Af, Gf, seed, layer, shared, signs, accum, n_sq, ws, s, mk);
    case DP_NORM_HUTCHPP:
      if (P.mfma) return run_norm_mfma_hpp(P, B, T, d, p, Ab, Gb, seed, layer, shared, signs, accum, n_sq, ws, s, mk);
      return bf ? run_norm_generic_hpp<bf16_t>(P, B, T, d, p, Ab, Gb, seed, layer, shared, signs, accum, n_sq, ws, s, mk)
                : run_norm_generic_hpp<float>(P, B, T, d, p, Af, Gf, seed, layer, shared, signs, accum, n_sq, ws, s, mk);
    default:
      return bf ? run_norm_exact<bf16_t>(method, P, B, T, d, p, Ab, Gb, accum, n_sq, ws, s, mk)
                : run_norm_exact<float>(method, P, B, T, d, p, Af, Gf, accum, n_sq, ws, s, mk);
  }
}

dp_status_t dp_norm_est(int method, int dtype, int B, int T, int d, int p, int k, const void* A,
                        const void* G, uint64_t seed, uint32_t layer, uint32_t flags, float* n_sq,
                        void* ws, size_t ws_bytes, dp_stream_t stream) {
  return norm_est_impl(method, dtype, B, T, d, p, k, A, G, seed, layer, flags, n_sq, ws, ws_bytes,
                       stream, Marks{});
}

dp_status_t dp_norm_est_timed(int method, int dtype, int B, int T, int d, int p, int k,
                              const void* A, const void* G, uint64_t seed, uint32_t layer,
                              uint32_t flags, float* n_sq, void* ws, size_t ws_bytes,
                              dp_stream_t stream, void* ev_begin, void* ev_end) {
  return norm_est_impl(method, dtype, B, T, d, p, k, A, G, seed, layer, flags, n_sq, ws, ws_bytes,
                       stream,
                       Marks{static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end)});
}

// ---- dp_norm_est_noalloc: the same call on a library-owned scratch array ----
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol): the device address is looked up
// once per device with hipGetSymbolAddress and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[DP_NOALLOC_SCRATCH_BYTES];

static std::mutex scratch_mu;
static void* scratch_ptr[kMaxDevices];  // per-device address of `scratch`, set once

static dp_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DP_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return DP_ERR_HIP;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return DP_OK;
}

dp_status_t dp_norm_est_noalloc(int method, int dtype, int B, int T, int d, int p, int k,
                                const void* A, const void* G, uint64_t seed, uint32_t layer,
                                uint32_t flags, float* n_sq, dp_stream_t stream) {
  if (!norm_args_ok(method, dtype, B, T, d, p, k)) return DP_ERR_INVALID_ARG;
  if (plan_norm(method, dtype, B, T, d, p, k).total > DP_NOALLOC_SCRATCH_BYTES)
    return DP_ERR_WORKSPACE;
  void* ws = nullptr;
  const dp_status_t st = scratch_address(&ws);
  if (st != DP_OK) return st;
  return norm_est_impl(method, dtype, B, T, d, p, k, A, G, seed, layer, flags, n_sq, ws,
                       DP_NOALLOC_SCRATCH_BYTES, stream, Marks{});
}

size_t dp_clip_aggregate_workspace(int dtype, int B, int T, int d, int p) {
  if (!agg_args_ok(dtype, B, T, d, p)) return kInvalid;
  return plan_agg(dtype, B, T, d, p).total;
}

int dp_norm_est_uses_mfma(int method, int dtype, int B, int T, int d, int p, int k) {
  if (!norm_args_ok(method, dtype, B, T, d, p, k)) return -1;
  return plan_norm(method, dtype, B, T, d, p, k).mfma ? 1 : 0;
}

int dp_clip_aggregate_uses_mfma(int dtype, int B, int T, int d, int p) {
  if (!agg_args_ok(dtype, B, T, d, p)) return -1;
  return plan_agg(dtype, B, T, d, p).mfma ? 1 : 0;
}

bool agg_ptrs_ok(int B, int T, const void* A, const void* G, const float* n_sq, float C,
                 float* c_out) {
  if (!(C > 0.f) || !std::isfinite(C)) return false;
  if (B > 0 && (n_sq == nullptr || !aligned(n_sq, 4))) return false;
  if (B > 0 && T > 0 && (A == nullptr || G == nullptr || !aligned(A, 16) || !aligned(G, 16)))
    return false;
  if (c_out && !aligned(c_out, 4)) return false;
  return true;
}

// Clip factors, then the clipped sum: into S directly (nsplit == 1 or the
// generic kernel), or as *nsplit planes at *planes (the workspace).  Returns
// where the sum is and how many planes make it up.
dp_status_t clip_and_sum(const AggPlan& P, int dtype, int B, int T, int d, int p, const void* A,
                         const void* G, const float* n_sq, float C, float* c_out, float* S,
                         void* ws, hipStream_t s, const Marks& mk, const float** planes,
                         int* nplanes, bool run_clip = true) {
  float* c = at<float>(ws, P.c);
  int* order = at<int>(ws, P.order);
  int* count = at<int>(ws, P.count);
  if (run_clip)  // else c, order and count are already in the workspace (batched call)
    DP_TRY(launch_clip(n_sq, B, C, c, c_out, at<uint32_t>(ws, P.status), order, count, s));
  *planes = S;
  *nplanes = 1;
  if (P.mfma) {
    const bf16_t* Ab = static_cast<const bf16_t*>(A);
    const bf16_t* Gb = static_cast<const bf16_t*>(G);
    float* dst = P.nsplit == 1 ? S : at<float>(ws, P.part);
    DP_TRY(mk.open(s));
    DP_TRY(launch_aggregate_mfma(Ab, Gb, B, T, d, p, c, order, count, P.nsplit, dst, s));
    DP_TRY(mk.close(s));
    *planes = dst;
    *nplanes = P.nsplit;
    return DP_OK;
  }
  DP_TRY(mk.open(s));
  if (dtype == DP_BF16) {
    DP_TRY(launch_aggregate_generic<bf16_t>(static_cast<const bf16_t*>(A),
                                            static_cast<const bf16_t*>(G), B, T, d, p, c, S, s));
  } else {
    DP_TRY(launch_aggregate_generic<float>(static_cast<const float*>(A),
                                           static_cast<const float*>(G), B, T, d, p, c, S, s));
  }
  DP_TRY(mk.close(s));
  return DP_OK;
}

static dp_status_t clip_aggregate_impl(int dtype, int B, int T, int d, int p, const void* A,
                                       const void* G, const float* n_sq, float C, float* c_out,
                                       float* S, void* ws, size_t ws_bytes, dp_stream_t stream,
                                       const Marks& mk) {
  if (!agg_args_ok(dtype, B, T, d, p)) return DP_ERR_INVALID_ARG;
  if (!agg_ptrs_ok(B, T, A, G, n_sq, C, c_out)) return DP_ERR_INVALID_ARG;
  if (S == nullptr || !aligned(S, 16)) return DP_ERR_INVALID_ARG;
  const AggPlan P = plan_agg(dtype, B, T, d, p);
  if (ws_bytes < P.total) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* planes = nullptr;
  int nplanes = 1;
  const dp_status_t st =
      clip_and_sum(P, dtype, B, T, d, p, A, G, n_sq, C, c_out, S, ws, s, mk, &planes, &nplanes);
  if (st != DP_OK) return st;
  if (planes != S) DP_TRY(launch_reduce_splits(planes, nplanes, static_cast<int64_t>(p) * d, S, s));
  return DP_OK;
}

// Whether [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool update_args_ok(int d, int p, int B, float sigma, float C, float eta) {
  if (d < 1 || p < 1 || B < 1) return false;
  return sigma >= 0.f && std::isfinite(sigma) && C > 0.f && std::isfinite(C) && std::isfinite(eta);
}

// One layer's clipped sum, noise and update on a validated plan.  run_clip =
// false: the clip factors are already in the workspace (batched call).
static dp_status_t aggregate_update_layer(const AggPlan& P, int dtype, int B, int T, int d, int p,
                                          const void* A, const void* G, const float* n_sq,
                                          float C, float sigma, float eta, uint64_t seed,
                                          uint32_t layer, float* theta, float* S, float* c_out,
                                          void* ws, hipStream_t s, const Marks& mk_agg,
                                          const Marks& mk_upd, bool run_clip) {
  float* sum = S != nullptr ? S : at<float>(ws, P.sbuf);
  const float* planes = nullptr;
  int nplanes = 1;
  const dp_status_t st = clip_and_sum(P, dtype, B, T, d, p, A, G, n_sq, C, c_out, sum, ws, s,
                                      mk_agg, &planes, &nplanes, run_clip);
  if (st != DP_OK) return st;
  const float sigmaC = sigma * C;
  const float eta_over_B = static_cast<float>(static_cast<double>(eta) / B);
  const int64_t n = static_cast<int64_t>(p) * d;
  DP_TRY(mk_upd.open(s));
  if (planes == sum)
    DP_TRY(launch_noise_update(theta, sum, n, sigmaC, eta_over_B, seed, layer, s));
  else
    DP_TRY(launch_noise_update_splits(theta, planes, nplanes, n, S, sigmaC, eta_over_B, seed,
                                      layer, s));
  DP_TRY(mk_upd.close(s));
  return DP_OK;
}

static dp_status_t clip_aggregate_update_impl(int dtype, int B, int T, int d, int p,
                                              const void* A, const void* G, const float* n_sq,
                                              float C, float sigma, float eta, uint64_t seed,
                                              uint32_t layer, float* theta, float* S,
                                              float* c_out, void* ws, size_t ws_bytes,
                                              dp_stream_t stream, const Marks& mk_agg,
                                              const Marks& mk_upd) {
  if (!agg_args_ok(dtype, B, T, d, p)) return DP_ERR_INVALID_ARG;
  if (!update_args_ok(d, p, B, sigma, C, eta)) return DP_ERR_INVALID_ARG;
  if (!agg_ptrs_ok(B, T, A, G, n_sq, C, c_out)) return DP_ERR_INVALID_ARG;
  if (theta == nullptr || !aligned(theta, 16)) return DP_ERR_INVALID_ARG;
  if (S != nullptr && !aligned(S, 16)) return DP_ERR_INVALID_ARG;
  const size_t bytes = static_cast<size_t>(p) * d * 4;
  if (S != nullptr && overlaps(theta, bytes, S, bytes)) return DP_ERR_INVALID_ARG;
  const AggPlan P = plan_agg(dtype, B, T, d, p, true);
  if (ws_bytes < P.total) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  if (overlaps(theta, bytes, ws, P.total) || (S != nullptr && overlaps(S, bytes, ws, P.total)))
    return DP_ERR_INVALID_ARG;
  return aggregate_update_layer(P, dtype, B, T, d, p, A, G, n_sq, C, sigma, eta, seed, layer,
                                theta, S, c_out, ws, static_cast<hipStream_t>(stream), mk_agg,
                                mk_upd, true);
}

dp_status_t dp_clip_aggregate(int dtype, int B, int T, int d, int p, const void* A, const void* G,
                              const float* n_sq, float C, float* c_out, float* S, void* ws,
                              size_t ws_bytes, dp_stream_t stream) {
  return clip_aggregate_impl(dtype, B, T, d, p, A, G, n_sq, C, c_out, S, ws, ws_bytes, stream,
                             Marks{});
}

dp_status_t dp_clip_aggregate_timed(int dtype, int B, int T, int d, int p, const void* A,
                                    const void* G, const float* n_sq, float C, float* c_out,
                                    float* S, void* ws, size_t ws_bytes, dp_stream_t stream,
                                    void* ev_begin, void* ev_end) {
  return clip_aggregate_impl(dtype, B, T, d, p, A, G, n_sq, C, c_out, S, ws, ws_bytes, stream,
                             Marks{static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end)});
}

static dp_status_t noise_update_impl(int d, int p, float* theta, const float* S, float sigma,
                                     float C, float eta, int B, uint64_t seed, uint32_t layer,
                                     dp_stream_t stream, const Marks& mk) {
  if (!update_args_ok(d, p, B, sigma, C, eta)) return DP_ERR_INVALID_ARG;
  if (theta == nullptr || S == nullptr || !aligned(theta, 16) || !aligned(S, 16))
    return DP_ERR_INVALID_ARG;
  const int64_t n = static_cast<int64_t>(p) * d;
  if (overlaps(theta, static_cast<size_t>(n) * 4, S, static_cast<size_t>(n) * 4))
    return DP_ERR_INVALID_ARG;
  const float sigmaC = sigma * C;
  const float eta_over_B = static_cast<float>(static_cast<double>(eta) / B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  DP_TRY(mk.open(s));
  DP_TRY(launch_noise_update(theta, S, n, sigmaC, eta_over_B, seed, layer, s));
  DP_TRY(mk.close(s));
  return DP_OK;
}

size_t dp_clip_aggregate_update_workspace(int dtype, int B, int T, int d, int p) {
  if (!agg_args_ok(dtype, B, T, d, p)) return kInvalid;
  return plan_agg(dtype, B, T, d, p, true).total;
}

dp_status_t dp_clip_aggregate_update(int dtype, int B, int T, int d, int p, const void* A,
                                     const void* G, const float* n_sq, float C, float sigma,
                                     float eta, uint64_t seed, uint32_t layer, float* theta,
                                     float* S, float* c_out, void* ws, size_t ws_bytes,
                                     dp_stream_t stream) {
  return clip_aggregate_update_impl(dtype, B, T, d, p, A, G, n_sq, C, sigma, eta, seed, layer,
                                    theta, S, c_out, ws, ws_bytes, stream, Marks{}, Marks{});
}

dp_status_t dp_clip_aggregate_update_timed(int dtype, int B, int T, int d, int p, const void* A,
                                           const void* G, const float* n_sq, float C,
                                           float sigma, float eta, uint64_t seed, uint32_t layer,
                                           float* theta, float* S, float* c_out, void* ws,
                                           size_t ws_bytes, dp_stream_t stream,
                                           void* ev_agg_begin, void* ev_agg_end,
                                           void* ev_upd_begin, void* ev_upd_end) {
  return clip_aggregate_update_impl(
      dtype, B, T, d, p, A, G, n_sq, C, sigma, eta, seed, layer, theta, S, c_out, ws, ws_bytes,
      stream,
      Marks{static_cast<hipEvent_t>(ev_agg_begin), static_cast<hipEvent_t>(ev_agg_end)},
      Marks{static_cast<hipEvent_t>(ev_upd_begin), static_cast<hipEvent_t>(ev_upd_end)});
}

dp_status_t dp_noise_update(int d, int p, float* theta, const float* S, float sigma, float C,
                            float eta, int B, uint64_t seed, uint32_t layer, dp_stream_t stream) {
  return noise_update_impl(d, p, theta, S, sigma, C, eta, B, seed, layer, stream, Marks{});
}

dp_status_t dp_noise_update_timed(int d, int p, float* theta, const float* S, float sigma, float C,
                                  float eta, int B, uint64_t seed, uint32_t layer,
                                  dp_stream_t stream, void* ev_begin, void* ev_end) {
  return noise_update_impl(d, p, theta, S, sigma, C, eta, B, seed, layer, stream,
                           Marks{static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end)});
}

dp_status_t dp_read_device_status(void* ws, uint32_t* flags_out, dp_stream_t stream) {
  if (ws == nullptr || flags_out == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* w = static_cast<uint32_t*>(ws);
  uint32_t v = 0;
  DP_TRY(launch_take_status(w, s));
  DP_TRY(hipMemcpyAsync(&v, w + 1, sizeof(v), hipMemcpyDeviceToHost, s));
  DP_TRY(hipStreamSynchronize(s));
  *flags_out = v;
  return DP_OK;
}

dp_status_t dp_stream_read(const void* buf, size_t bytes, uint32_t* out, int nblocks,
                           dp_stream_t stream) {
  if (bytes == 0) return DP_OK;
  if (buf == nullptr || out == nullptr || !aligned(buf, 16) || !aligned(out, 4) || bytes % 16 != 0 ||
      nblocks < 1 || nblocks > 65536)
    return DP_ERR_INVALID_ARG;
  DP_TRY(launch_stream_read(buf, static_cast<int64_t>(bytes / 16), out, nblocks,
                            static_cast<hipStream_t>(stream)));
  return DP_OK;
}

dp_status_t dp_philox_u32(uint64_t seed, const uint32_t* ctr, uint32_t* out, size_t n,
                          dp_stream_t stream) {
  if (n == 0) return DP_OK;
  if (ctr == nullptr || out == nullptr || !aligned(ctr, 4) || !aligned(out, 4))
    return DP_ERR_INVALID_ARG;
  DP_TRY(launch_philox_u32(seed, ctr, out, n, static_cast<hipStream_t>(stream)));
  return DP_OK;
}

dp_status_t dp_probe_fill(uint64_t seed, uint32_t layer, uint32_t sample, int p, int k, float* Pt,
                          dp_stream_t stream) {
  if (p < 1 || k < 1 || Pt == nullptr || !aligned(Pt, 4)) return DP_ERR_INVALID_ARG;
  DP_TRY(launch_probe_fill_f32(seed, layer, sample, 1, p, k, k, Pt,
                               static_cast<hipStream_t>(stream)));
  return DP_OK;
}

dp_status_t dp_probe_fill_ex(uint64_t seed, uint32_t layer, uint32_t sample, int p, int k,
                             uint32_t flags, float* Pt, dp_stream_t stream) {
  if ((flags & ~DP_PROBE_RADEMACHER) != 0) return DP_ERR_INVALID_ARG;
  if (p < 1 || k < 1 || Pt == nullptr || !aligned(Pt, 4)) return DP_ERR_INVALID_ARG;
  DP_TRY(launch_probe_fill_f32(seed, layer, sample, 1, p, k, k, Pt,
                               static_cast<hipStream_t>(stream),
                               (flags & DP_PROBE_RADEMACHER) != 0));
  return DP_OK;
}

dp_status_t dp_noise_fill(uint64_t seed, uint32_t layer, uint64_t offset, size_t n, float* xi,
                          dp_stream_t stream) {
  if (n == 0) return DP_OK;
  if (xi == nullptr || !aligned(xi, 4)) return DP_ERR_INVALID_ARG;
  if (offset + n < offset) return DP_ERR_INVALID_ARG;
  DP_TRY(launch_noise_fill(seed, layer, offset, n, xi, static_cast<hipStream_t>(stream)));
  return DP_OK;
}

size_t dp_poisson_sample_workspace(int64_t N) {
  if (N < 0 || N > (static_cast<int64_t>(1) << 40)) return kInvalid;
  const int64_t nblk = poisson_blocks(N);
  return static_cast<size_t>(nblk > 0 ? nblk : 1) * sizeof(int64_t);
}

dp_status_t dp_poisson_sample(uint64_t seed, uint32_t step, int64_t N, double q, int64_t* idx,
                              int64_t idx_cap, int64_t* count, void* ws, size_t ws_bytes,
                              dp_stream_t stream) {
  const size_t need = dp_poisson_sample_workspace(N);
  if (need == kInvalid || !(q >= 0.0 && q <= 1.0) || idx_cap < 0) return DP_ERR_INVALID_ARG;
  if (count == nullptr || !aligned(count, 8)) return DP_ERR_INVALID_ARG;
  if (idx_cap > 0 && (idx == nullptr || !aligned(idx, 8))) return DP_ERR_INVALID_ARG;
  if (ws_bytes < need) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  // floor(q 2^32): scaling a double by 2^32 is exact, and so is the floor
  const uint64_t thr = static_cast<uint64_t>(std::floor(q * 4294967296.0));
  DP_TRY(launch_poisson_sample(seed, step, N, thr, idx, idx_cap, count, static_cast<int64_t*>(ws),
                               static_cast<hipStream_t>(stream)));
  return DP_OK;
}

// ---- RMSNorm gains ----
// [part: B][nsplit][d] fp32 | [sq: B][chunks] fp64
static size_t rmsnorm_part_bytes(int B, int T, int d) {
  return align_up(static_cast<size_t>(B) * rmsnorm_splits(B, T, d) * d * sizeof(float) + 16);
}

size_t dp_rmsnorm_norm_workspace(int dtype, int B, int T, int d) {
  if (!valid_dtype(dtype) || B < 0 || T < 0 || d < 1) return kInvalid;
  return rmsnorm_part_bytes(B, T, d) +
         align_up(static_cast<size_t>(B > 0 ? B : 1) * rmsnorm_sq_chunks(d) * sizeof(double));
}

dp_status_t dp_rmsnorm_norm(int dtype, int B, int T, int d, const void* xhat, const void* delta,
                            uint32_t flags, float* n_sq, float* v, void* ws, size_t ws_bytes,
                            dp_stream_t stream) {
  const size_t need = dp_rmsnorm_norm_workspace(dtype, B, T, d);
  if (need == kInvalid || (flags & ~DP_ACCUMULATE) != 0) return DP_ERR_INVALID_ARG;
  if (B == 0) return DP_OK;
  if (n_sq == nullptr || !aligned(n_sq, 4) || (v != nullptr && !aligned(v, 4)))
    return DP_ERR_INVALID_ARG;
  if (T > 0 && (xhat == nullptr || delta == nullptr || !aligned(xhat, 16) || !aligned(delta, 16)))
    return DP_ERR_INVALID_ARG;
  if (ws_bytes < need) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nsplit = rmsnorm_splits(B, T, d);
  const int acc = (flags & DP_ACCUMULATE) ? 1 : 0;
  double* sq = at<double>(ws, rmsnorm_part_bytes(B, T, d));
  if (dtype == DP_BF16)
    DP_TRY(launch_rmsnorm_norm(static_cast<const bf16_t*>(xhat), static_cast<const bf16_t*>(delta),
                               B, T, d, static_cast<float*>(ws), nsplit, sq, v, n_sq, acc, s));
  else
    DP_TRY(launch_rmsnorm_norm(static_cast<const float*>(xhat), static_cast<const float*>(delta),
                               B, T, d, static_cast<float*>(ws), nsplit, sq, v, n_sq, acc, s));
  return DP_OK;
}

struct GainPlan {
  size_t status = 0, c = 0, order = 0, count = 0, sbuf = 0, total = 0;
};

static GainPlan plan_gain(int B, int d) {
  GainPlan P;
  Carver cv;
  const size_t Bz = static_cast<size_t>(B > 0 ? B : 1);
  P.status = cv.take(kStatusBytes);
  P.c = cv.take(Bz * sizeof(float));
  P.order = cv.take(Bz * sizeof(int));
  P.count = cv.take(sizeof(int));
  P.sbuf = cv.take(static_cast<size_t>(d) * sizeof(float));
  P.total = cv.off;
  return P;
}

size_t dp_rmsnorm_update_workspace(int B, int d) {
  if (B < 1 || d < 1) return kInvalid;
  return plan_gain(B, d).total;
}

dp_status_t dp_rmsnorm_clip_aggregate_update(int B, int d, const float* v, const float* n_sq,
                                             float C, float sigma, float eta, uint64_t seed,
                                             uint32_t layer, float* gamma, float* S,
                                             float* c_out, void* ws, size_t ws_bytes,
                                             dp_stream_t stream) {
  if (!update_args_ok(d, 1, B, sigma, C, eta)) return DP_ERR_INVALID_ARG;
  if (v == nullptr || n_sq == nullptr || gamma == nullptr || !aligned(v, 4) ||
      !aligned(n_sq, 4) || !aligned(gamma, 16))
    return DP_ERR_INVALID_ARG;
  if ((S != nullptr && !aligned(S, 16)) || (c_out && !aligned(c_out, 4))) return DP_ERR_INVALID_ARG;
  const size_t bytes = static_cast<size_t>(d) * 4;
  if (S != nullptr && overlaps(gamma, bytes, S, bytes)) return DP_ERR_INVALID_ARG;
  const GainPlan P = plan_gain(B, d);
  if (ws_bytes < P.total) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  if (overlaps(gamma, bytes, ws, P.total)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* c = at<float>(ws, P.c);
  float* sum = S != nullptr ? S : at<float>(ws, P.sbuf);
  DP_TRY(launch_clip(n_sq, B, C, c, c_out, at<uint32_t>(ws, P.status), at<int>(ws, P.order),
                     at<int>(ws, P.count), s));
  DP_TRY(launch_weighted_rows(v, c, B, d, sum, s));
  const float eta_over_B = static_cast<float>(static_cast<double>(eta) / B);
  DP_TRY(launch_noise_update(gamma, sum, d, sigma * C, eta_over_B, seed, layer, s));
  return DP_OK;
}

// ---- embedding tables ----
constexpr int kEmbMaxTokens = 16384;

struct EmbPlan {
  int nsplit = 1, nchunk = 1;
  size_t status = 0, spos = 0, sid = 0, gidp = 0, ustart = 0, uid = 0, ng = 0, head = 0, tail = 0, part = 0,
         cpart = 0, gsum = 0, rowmap = 0, c = 0, order = 0, count = 0, total = 0;
};

static EmbPlan plan_emb(int B, int T, int d, int V) {
  EmbPlan P;
  Carver cv;
  const size_t Bz = static_cast<size_t>(B > 0 ? B : 1), Tz = static_cast<size_t>(T > 0 ? T : 1);
  P.nsplit = emb_splits(B, T, d);
  P.nchunk = (d + 2047) / 2048;
  if (V > 0) P.status = cv.take(kStatusBytes);  // the update forms clip factors
  P.spos = cv.take(Bz * Tz * 4);
  P.sid = cv.take(Bz * Tz * 4);
  P.gidp = cv.take(Bz * Tz * 4);
  P.ustart = cv.take(Bz * (Tz + 1) * 4);
  P.uid = cv.take(Bz * Tz * 4);
  P.ng = cv.take(Bz * 4);
  P.head = cv.take(Bz * P.nsplit * static_cast<size_t>(d) * 4);
  P.tail = cv.take(Bz * P.nsplit * static_cast<size_t>(d) * 4);
  if (V == 0) {
    P.part = cv.take(Bz * P.nsplit * P.nchunk * sizeof(double));
    P.cpart = cv.take(Bz * emb_combine_chunks(d) * sizeof(double));
  } else {
    P.gsum = cv.take(Bz * Tz * static_cast<size_t>(d) * 4);
    P.rowmap = cv.take(Bz * static_cast<size_t>(V) * 4);
    P.c = cv.take(Bz * sizeof(float));
    P.order = cv.take(Bz * sizeof(int));
    P.count = cv.take(sizeof(int));
  }
  P.total = cv.off;
  return P;
}

static bool emb_args_ok(int dtype, int B, int T, int d) {
  return valid_dtype(dtype) && B >= 0 && T >= 0 && T <= kEmbMaxTokens && d >= 1;
}

size_t dp_embedding_norm_workspace(int dtype, int B, int T, int d) {
  if (!emb_args_ok(dtype, B, T, d)) return kInvalid;
  return plan_emb(B, T, d, 0).total;
}

dp_status_t dp_embedding_norm(int dtype, int B, int T, int d, const int32_t* ids,
                              const void* delta, uint32_t flags, float* n_sq, void* ws,
                              size_t ws_bytes, dp_stream_t stream) {
  if (!emb_args_ok(dtype, B, T, d) || (flags & ~DP_ACCUMULATE) != 0) return DP_ERR_INVALID_ARG;
  if (B == 0) return DP_OK;
  if (n_sq == nullptr || !aligned(n_sq, 4)) return DP_ERR_INVALID_ARG;
  if (T > 0 && (ids == nullptr || delta == nullptr || !aligned(ids, 4) || !aligned(delta, 16)))
    return DP_ERR_INVALID_ARG;
  const EmbPlan P = plan_emb(B, T, d, 0);
  if (ws_bytes < P.total) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int acc = (flags & DP_ACCUMULATE) ? 1 : 0;
  if (T == 0) {
    DP_TRY(launch_emb_zero_norm(B, n_sq, acc, s));
    return DP_OK;
  }
  int32_t* spos = at<int32_t>(ws, P.spos);
  int32_t* sid = at<int32_t>(ws, P.sid);
  int32_t* gidp = at<int32_t>(ws, P.gidp);
  DP_TRY(launch_emb_sort(ids, B, T, spos, sid, gidp, at<int32_t>(ws, P.ustart),
                         at<int32_t>(ws, P.uid), at<int32_t>(ws, P.ng), s));
  double* part = at<double>(ws, P.part);
  double* cpart = at<double>(ws, P.cpart);
  float* head = at<float>(ws, P.head);
  float* tail = at<float>(ws, P.tail);
  if (dtype == DP_BF16)
    DP_TRY(launch_emb_norm(static_cast<const bf16_t*>(delta), B, T, d, spos, sid, gidp, P.nsplit,
                           part, head, tail, cpart, n_sq, acc, s));
  else
    DP_TRY(launch_emb_norm(static_cast<const float*>(delta), B, T, d, spos, sid, gidp, P.nsplit,
                           part, head, tail, cpart, n_sq, acc, s));
  return DP_OK;
}

size_t dp_embedding_update_workspace(int dtype, int B, int T, int d, int V) {
  if (!emb_args_ok(dtype, B, T, d) || B < 1 || V < 1) return kInvalid;
  return plan_emb(B, T, d, V).total;
}

dp_status_t dp_embedding_clip_aggregate_update(int dtype, int B, int T, int d, int V,
                                               const int32_t* ids, const void* delta,
                                               const float* n_sq, float C, float sigma,
                                               float eta, uint64_t seed, uint32_t layer, float* E,
                                               float* c_out, void* ws, size_t ws_bytes,
                                               dp_stream_t stream) {
  if (!emb_args_ok(dtype, B, T, d) || V < 1) return DP_ERR_INVALID_ARG;
  if (!update_args_ok(d, V, B, sigma, C, eta)) return DP_ERR_INVALID_ARG;
  if (n_sq == nullptr || E == nullptr || !aligned(n_sq, 4) || !aligned(E, 16))
    return DP_ERR_INVALID_ARG;
  if (T > 0 && (ids == nullptr || delta == nullptr || !aligned(ids, 4) || !aligned(delta, 16)))
    return DP_ERR_INVALID_ARG;
  if (c_out && !aligned(c_out, 4)) return DP_ERR_INVALID_ARG;
  const EmbPlan P = plan_emb(B, T, d, V);
  if (ws_bytes < P.total) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  if (overlaps(E, static_cast<size_t>(V) * d * 4, ws, P.total)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* c = at<float>(ws, P.c);
  DP_TRY(launch_clip(n_sq, B, C, c, c_out, at<uint32_t>(ws, P.status), at<int>(ws, P.order),
                     at<int>(ws, P.count), s));
  int32_t* spos = at<int32_t>(ws, P.spos);
  int32_t* sid = at<int32_t>(ws, P.sid);
  int32_t* gidp = at<int32_t>(ws, P.gidp);
  int32_t* uid = at<int32_t>(ws, P.uid);
  int32_t* ng = at<int32_t>(ws, P.ng);
  float* gsum = at<float>(ws, P.gsum);
  if (T > 0) {
    DP_TRY(launch_emb_sort(ids, B, T, spos, sid, gidp, at<int32_t>(ws, P.ustart), uid, ng, s));
    if (dtype == DP_BF16)
      DP_TRY(launch_emb_group_sums(static_cast<const bf16_t*>(delta), B, T, d, spos, sid, gidp,
                                   P.nsplit, at<float>(ws, P.head), at<float>(ws, P.tail), gsum,
                                   s));
    else
      DP_TRY(launch_emb_group_sums(static_cast<const float*>(delta), B, T, d, spos, sid, gidp,
                                   P.nsplit, at<float>(ws, P.head), at<float>(ws, P.tail), gsum,
                                   s));
  }
  const float eta_over_B = static_cast<float>(static_cast<double>(eta) / B);
  DP_TRY(launch_emb_update(gsum, B, T, d, uid, ng, at<int32_t>(ws, P.rowmap), V, c, E, sigma * C,
                           eta_over_B, seed, layer, s));
  return DP_OK;
}

// ---- MLP block: forward pass and backward pass 1 ----

struct Region {
  const void* p;
  size_t n;
};

// True if two of the outputs overlap, or an output overlaps an input (an
// output equal to an input pointer with the same size is allowed only where
// the caller marks it with `same`).
static bool regions_clash(const Region* outs, int no, const Region* ins, int ni,
                          const void* same_out = nullptr, const void* same_in = nullptr) {
  for (int a = 0; a < no; ++a) {
    for (int b = a + 1; b < no; ++b)
      if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return true;
    for (int b = 0; b < ni; ++b) {
      if (outs[a].p == same_out && ins[b].p == same_in && same_out != nullptr) continue;
      if (overlaps(outs[a].p, outs[a].n, ins[b].p, ins[b].n)) return true;
    }
  }
  return false;
}

static bool mlp_dims_ok(int B, int T, int d, int f) {
  if (B < 0 || T < 0 || d < 256 || f < 256 || d % 256 != 0 || f % 256 != 0) return false;
  return static_cast<int64_t>(B) * T <= (int64_t{1} << 30);
}

static bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr || !aligned(p, 16)) return false;
  return true;
}

dp_status_t dp_weights_bf16(int p, int d, const float* theta, void* W, void* Wt,
                            dp_stream_t stream) {
  if (p < 0 || d < 0 || p % 64 != 0 || d % 64 != 0) return DP_ERR_INVALID_ARG;
  if (p == 0 || d == 0) return DP_OK;
  if (!all_aligned16({theta, W}) || Wt == nullptr || !aligned(Wt, 8)) return DP_ERR_INVALID_ARG;
  const size_t n = static_cast<size_t>(p) * d;
  const Region outs[] = {{W, n * 2}, {Wt, n * 2}};
  const Region ins[] = {{theta, n * 4}};
  if (regions_clash(outs, 2, ins, 1)) return DP_ERR_INVALID_ARG;
  DP_TRY(launch_cast_transpose(theta, p, d, static_cast<bf16_t*>(W), static_cast<bf16_t*>(Wt),
                               static_cast<hipStream_t>(stream)));
  return DP_OK;
}

dp_status_t dp_linear_forward(int64_t M, int N, int K, const void* A, const void* W,
                              const void* residual, void* C, dp_stream_t stream) {
  if (M < 0 || M > (int64_t{1} << 30) || N <= 0 || N % 256 != 0 || K <= 0 || K % 32 != 0)
    return DP_ERR_INVALID_ARG;
  if (M == 0) return DP_OK;
  if (!all_aligned16({A, W}) || C == nullptr || !aligned(C, 8) ||
      (residual != nullptr && !aligned(residual, 8)))
    return DP_ERR_INVALID_ARG;
  const size_t mn = static_cast<size_t>(M) * N * 2;
  const Region outs[] = {{C, mn}};
  const Region ins[] = {{A, static_cast<size_t>(M) * K * 2}, {W, static_cast<size_t>(N) * K * 2},
                        {residual, residual ? mn : 0}};
  if (regions_clash(outs, 1, ins, 3, C, residual)) return DP_ERR_INVALID_ARG;
  DP_TRY(launch_gemm_nt(static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(W), K, nullptr,
                        nullptr, 0, M, N, static_cast<const bf16_t*>(residual),
                        static_cast<bf16_t*>(C), static_cast<hipStream_t>(stream)));
  return DP_OK;
}

dp_status_t dp_mlp_forward(int B, int T, int d, int f, float eps, const void* x,
                           const float* gamma, const void* Wg, const void* Wu, const void* Wd,
                           void* xhat, void* y, float* rstd, void* g, void* u, void* h, void* out,
                           dp_stream_t stream) {
  if (!mlp_dims_ok(B, T, d, f) || !(eps >= 0.f) || !std::isfinite(eps)) return DP_ERR_INVALID_ARG;
  const int64_t M = static_cast<int64_t>(B) * T;
  if (M == 0) return DP_OK;
  if (!all_aligned16({x, gamma, Wg, Wu, Wd, xhat, y, g, u, h, out}) || rstd == nullptr ||
      !aligned(rstd, 4))
    return DP_ERR_INVALID_ARG;
  const size_t md = static_cast<size_t>(M) * d * 2, mf = static_cast<size_t>(M) * f * 2,
               w = static_cast<size_t>(d) * f * 2;
  const Region outs[] = {{xhat, md}, {y, md}, {rstd, static_cast<size_t>(M) * 4},
                         {g, mf},    {u, mf}, {h, mf},
                         {out, md}};
  const Region ins[] = {{x, md}, {gamma, static_cast<size_t>(d) * 4}, {Wg, w}, {Wu, w}, {Wd, w}};
  if (regions_clash(outs, 7, ins, 5, out, x)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  bf16_t* yb = static_cast<bf16_t*>(y);
  bf16_t* gb = static_cast<bf16_t*>(g);
  bf16_t* ub = static_cast<bf16_t*>(u);
  bf16_t* hb = static_cast<bf16_t*>(h);
  DP_TRY(launch_rmsnorm_fwd(xb, gamma, M, d, eps, static_cast<bf16_t*>(xhat), yb, rstd, s));
  // gate and up in one product; its epilogue writes g, u and h = silu(g) u
  DP_TRY(launch_gemm_nt_swiglu(yb, static_cast<const bf16_t*>(Wg), static_cast<const bf16_t*>(Wu),
                               d, M, f, gb, ub, hb, s));
  DP_TRY(launch_gemm_nt(hb, static_cast<const bf16_t*>(Wd), f, nullptr, nullptr, 0, M, d, xb,
                        static_cast<bf16_t*>(out), s));
  return DP_OK;
}

dp_status_t dp_mlp_backward(int B, int T, int d, int f, const void* x, const float* rstd,
                            const float* gamma, const void* g, const void* u, const void* WgT,
                            const void* WuT, const void* WdT, const void* dout, void* G_gate,
                            void* G_up, void* dy, void* dx, dp_stream_t stream) {
  if (!mlp_dims_ok(B, T, d, f)) return DP_ERR_INVALID_ARG;
  const int64_t M = static_cast<int64_t>(B) * T;
  if (M == 0) return DP_OK;
  if (!all_aligned16({x, gamma, g, u, WgT, WuT, WdT, dout, G_gate, G_up, dy, dx}) ||
      rstd == nullptr || !aligned(rstd, 4))
    return DP_ERR_INVALID_ARG;
  const size_t md = static_cast<size_t>(M) * d * 2, mf = static_cast<size_t>(M) * f * 2,
               w = static_cast<size_t>(d) * f * 2;
  const Region outs[] = {{G_gate, mf}, {G_up, mf}, {dy, md}, {dx, md}};
  const Region ins[] = {{x, md},   {rstd, static_cast<size_t>(M) * 4}, {gamma, static_cast<size_t>(d) * 4},
                        {g, mf},   {u, mf},
                        {WgT, w},  {WuT, w},
                        {WdT, w},  {dout, md}};
  if (regions_clash(outs, 4, ins, 9)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bf16_t* gg = static_cast<bf16_t*>(G_gate);
  bf16_t* gu = static_cast<bf16_t*>(G_up);
  const bf16_t* db = static_cast<const bf16_t*>(dout);
  // dh = R Wd stays in registers: the product's epilogue writes dL/dg and dL/du.
  DP_TRY(launch_gemm_nt_swiglu_bwd(db, static_cast<const bf16_t*>(WdT), d, M, f,
                                   static_cast<const bf16_t*>(g), static_cast<const bf16_t*>(u), gg,
                                   gu, s));
  // dy = G_gate Wg + G_up Wu: one product over the two k ranges.
  DP_TRY(launch_gemm_nt(gg, static_cast<const bf16_t*>(WgT), f, gu,
                        static_cast<const bf16_t*>(WuT), f, M, d, nullptr,
                        static_cast<bf16_t*>(dy), s));
  DP_TRY(launch_rmsnorm_bwd(static_cast<const bf16_t*>(x), rstd, gamma,
                            static_cast<const bf16_t*>(dy), db, M, d, static_cast<bf16_t*>(dx),
                            s));
  return DP_OK;
}


// ---- attention block: forward pass ----

static bool attn_dims_ok(int B, int T, int d, int H, int KV) {
  if (B < 0 || T < 0 || d < 256 || d % 256 != 0 || H < 1 || KV < 1 || H % KV != 0) return false;
  if ((H * 64) % 256 != 0 || (KV * 64) % 256 != 0) return false;
  if (T > 0 && !attn_shape_ok(T, H, KV)) return false;
  return static_cast<int64_t>(B) * T <= (int64_t{1} << 30);
}

dp_status_t dp_rope(int64_t M, int T, int n_heads, double base, int inverse, void* x,
                    dp_stream_t stream) {
  if (M < 0 || T < 1 || n_heads < 1 || !(base > 1.0) || !std::isfinite(base) ||
      (inverse != 0 && inverse != 1))
    return DP_ERR_INVALID_ARG;
  if (M == 0) return DP_OK;
  if (x == nullptr || !aligned(x, 16)) return DP_ERR_INVALID_ARG;
  DP_TRY(launch_rope(static_cast<bf16_t*>(x), M, T, n_heads, base, inverse != 0,
                     static_cast<hipStream_t>(stream)));
  return DP_OK;
}

dp_status_t dp_attention_forward(int B, int T, int H, int KV, const void* q, const void* k,
                                 const void* v, void* o, float* lse, dp_stream_t stream) {
  if (B < 0 || T < 0 || H < 1 || KV < 1 || H % KV != 0) return DP_ERR_INVALID_ARG;
  if (B == 0 || T == 0) return DP_OK;
  if (!attn_shape_ok(T, H, KV)) return DP_ERR_INVALID_ARG;
  if (!all_aligned16({q, k, v, o}) || lse == nullptr || !aligned(lse, 4)) return DP_ERR_INVALID_ARG;
  const size_t M = static_cast<size_t>(B) * T;
  const Region outs[] = {{o, M * H * 128}, {lse, M * H * 4}};
  const Region ins[] = {{q, M * H * 128}, {k, M * KV * 128}, {v, M * KV * 128}};
  if (regions_clash(outs, 2, ins, 3)) return DP_ERR_INVALID_ARG;
  DP_TRY(launch_attn_fwd(static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                         static_cast<const bf16_t*>(v), B, T, H, KV, static_cast<bf16_t*>(o), lse,
                         static_cast<hipStream_t>(stream)));
  return DP_OK;
}

dp_status_t dp_attn_forward(int B, int T, int d, int H, int KV, float eps, double rope_base,
                            const void* x, const float* gamma, const void* Wq, const void* Wk,
                            const void* Wv, const void* Wo, void* xhat, void* y, float* rstd,
                            void* q, void* k, void* v, void* o, float* lse, void* out,
                            dp_stream_t stream) {
  if (!attn_dims_ok(B, T, d, H, KV) || !(eps >= 0.f) || !std::isfinite(eps) ||
      !(rope_base > 1.0) || !std::isfinite(rope_base))
    return DP_ERR_INVALID_ARG;
  const int64_t M = static_cast<int64_t>(B) * T;
  if (M == 0) return DP_OK;
  if (!all_aligned16({x, gamma, Wq, Wk, Wv, Wo, xhat, y, q, k, v, o, out}) || rstd == nullptr ||
      !aligned(rstd, 4) || lse == nullptr || !aligned(lse, 4))
    return DP_ERR_INVALID_ARG;
  const int nq = H * 64, nk = KV * 64;
  const size_t md = static_cast<size_t>(M) * d * 2;
  const Region outs[] = {{xhat, md}, {y, md}, {rstd, static_cast<size_t>(M) * 4},
                         {q, static_cast<size_t>(M) * nq * 2}, {k, static_cast<size_t>(M) * nk * 2},
                         {v, static_cast<size_t>(M) * nk * 2}, {o, static_cast<size_t>(M) * nq * 2},
                         {lse, static_cast<size_t>(M) * H * 4}, {out, md}};
  const Region ins[] = {{x, md}, {gamma, static_cast<size_t>(d) * 4},
                        {Wq, static_cast<size_t>(nq) * d * 2}, {Wk, static_cast<size_t>(nk) * d * 2},
                        {Wv, static_cast<size_t>(nk) * d * 2}, {Wo, static_cast<size_t>(d) * nq * 2}};
  if (regions_clash(outs, 9, ins, 6, out, x)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  bf16_t* yb = static_cast<bf16_t*>(y);
  bf16_t* qb = static_cast<bf16_t*>(q);
  bf16_t* kb = static_cast<bf16_t*>(k);
  bf16_t* vb = static_cast<bf16_t*>(v);
  bf16_t* ob = static_cast<bf16_t*>(o);
  DP_TRY(launch_rmsnorm_fwd(xb, gamma, M, d, eps, static_cast<bf16_t*>(xhat), yb, rstd, s));
  DP_TRY(launch_gemm_nt(yb, static_cast<const bf16_t*>(Wq), d, nullptr, nullptr, 0, M, nq, nullptr,
                        qb, s));
  DP_TRY(launch_gemm_nt(yb, static_cast<const bf16_t*>(Wk), d, nullptr, nullptr, 0, M, nk, nullptr,
                        kb, s));
  DP_TRY(launch_gemm_nt(yb, static_cast<const bf16_t*>(Wv), d, nullptr, nullptr, 0, M, nk, nullptr,
                        vb, s));
  DP_TRY(launch_rope(qb, M, T, H, rope_base, false, s));
  DP_TRY(launch_rope(kb, M, T, KV, rope_base, false, s));
  DP_TRY(launch_attn_fwd(qb, kb, vb, B, T, H, KV, ob, lse, s));
  DP_TRY(launch_gemm_nt(ob, static_cast<const bf16_t*>(Wo), nq, nullptr, nullptr, 0, M, d, xb,
                        static_cast<bf16_t*>(out), s));
  return DP_OK;
}


// ---- attention block: backward pass 1 ----

size_t dp_attention_backward_workspace(int B, int T, int H) {
  if (B < 0 || T < 0 || H < 1) return kInvalid;
  return align_up(attn_bwd_scratch_bytes(B > 0 ? B : 1, T > 0 ? T : 1, H));
}

dp_status_t dp_attention_backward(int B, int T, int H, int KV, const void* q, const void* k,
                                  const void* v, const void* o, const float* lse, const void* dO,
                                  void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                                  dp_stream_t stream) {
  const size_t need = dp_attention_backward_workspace(B, T, H);
  if (need == kInvalid || KV < 1 || H % KV != 0) return DP_ERR_INVALID_ARG;
  if (B == 0 || T == 0) return DP_OK;
  if (!attn_shape_ok(T, H, KV)) return DP_ERR_INVALID_ARG;
  if (!all_aligned16({q, k, v, o, dO, dq, dk, dv}) || lse == nullptr || !aligned(lse, 4))
    return DP_ERR_INVALID_ARG;
  if (ws_bytes < need) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  const size_t M = static_cast<size_t>(B) * T;
  const Region outs[] = {{dq, M * H * 128}, {dk, M * KV * 128}, {dv, M * KV * 128}, {ws, need}};
  const Region ins[] = {{q, M * H * 128}, {k, M * KV * 128}, {v, M * KV * 128},
                        {o, M * H * 128}, {lse, M * H * 4},  {dO, M * H * 128}};
  if (regions_clash(outs, 4, ins, 6)) return DP_ERR_INVALID_ARG;
  DP_TRY(launch_attn_bwd(static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                         static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(o), lse,
                         static_cast<const bf16_t*>(dO), B, T, H, KV, static_cast<float*>(ws),
                         static_cast<bf16_t*>(dq), static_cast<bf16_t*>(dk),
                         static_cast<bf16_t*>(dv), static_cast<hipStream_t>(stream)));
  return DP_OK;
}

size_t dp_attn_backward_workspace(int B, int T, int H) {
  if (B < 0 || T < 0 || H < 1) return kInvalid;
  const size_t M = static_cast<size_t>(B > 0 ? B : 1) * (T > 0 ? T : 1);
  return align_up(M * H * 64 * 2) + dp_attention_backward_workspace(B, T, H);
}

dp_status_t dp_attn_backward(int B, int T, int d, int H, int KV, double rope_base, const void* x,
                             const float* rstd, const float* gamma, const void* q, const void* k,
                             const void* v, const void* o, const float* lse, const void* WqT,
                             const void* WkT, const void* WvT, const void* WoT, const void* dout,
                             void* G_q, void* G_k, void* G_v, void* dy, void* dx, void* ws,
                             size_t ws_bytes, dp_stream_t stream) {
  if (!attn_dims_ok(B, T, d, H, KV) || !(rope_base > 1.0) || !std::isfinite(rope_base))
    return DP_ERR_INVALID_ARG;
  const int64_t M = static_cast<int64_t>(B) * T;
  if (M == 0) return DP_OK;
  const size_t need = dp_attn_backward_workspace(B, T, H);
  if (!all_aligned16({x, gamma, q, k, v, o, WqT, WkT, WvT, WoT, dout, G_q, G_k, G_v, dy, dx}) ||
      rstd == nullptr || !aligned(rstd, 4) || lse == nullptr || !aligned(lse, 4))
    return DP_ERR_INVALID_ARG;
  if (ws_bytes < need) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  const int nq = H * 64, nk = KV * 64;
  const size_t md = static_cast<size_t>(M) * d * 2, mq = static_cast<size_t>(M) * nq * 2,
               mk = static_cast<size_t>(M) * nk * 2;
  const Region outs[] = {{G_q, mq}, {G_k, mk}, {G_v, mk}, {dy, md}, {dx, md}, {ws, need}};
  const Region ins[] = {{x, md},    {rstd, static_cast<size_t>(M) * 4}, {gamma, static_cast<size_t>(d) * 4},
                        {q, mq},    {k, mk},  {v, mk},  {o, mq},  {lse, static_cast<size_t>(M) * H * 4},
                        {WqT, static_cast<size_t>(nq) * d * 2}, {WkT, static_cast<size_t>(nk) * d * 2},
                        {WvT, static_cast<size_t>(nk) * d * 2}, {WoT, static_cast<size_t>(nq) * d * 2},
                        {dout, md}};
  if (regions_clash(outs, 6, ins, 13)) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bf16_t* dO = static_cast<bf16_t*>(ws);
  float* Dvec = at<float>(ws, align_up(mq));
  bf16_t* gq = static_cast<bf16_t*>(G_q);
  bf16_t* gk = static_cast<bf16_t*>(G_k);
  bf16_t* gv = static_cast<bf16_t*>(G_v);
  const bf16_t* db = static_cast<const bf16_t*>(dout);
  // dO = R Wo (the output gradient of the attention heads)
  DP_TRY(launch_gemm_nt(db, static_cast<const bf16_t*>(WoT), d, nullptr, nullptr, 0, M, nq, nullptr,
                        dO, s));
  DP_TRY(launch_attn_bwd(static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                         static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(o), lse, dO, B,
                         T, H, KV, Dvec, gq, gk, gv, s));
  // back through RoPE: the transpose of the rotation
  DP_TRY(launch_rope(gq, M, T, H, rope_base, true, s));
  DP_TRY(launch_rope(gk, M, T, KV, rope_base, true, s));
  // dy = G_q Wq + G_k Wk + G_v Wv: one product over three k ranges
  DP_TRY(launch_gemm_nt3(gq, static_cast<const bf16_t*>(WqT), nq, gk,
                         static_cast<const bf16_t*>(WkT), nk, gv, static_cast<const bf16_t*>(WvT),
                         nk, M, d, nullptr, static_cast<bf16_t*>(dy), s));
  DP_TRY(launch_rmsnorm_bwd(static_cast<const bf16_t*>(x), rstd, gamma,
                            static_cast<const bf16_t*>(dy), db, M, d, static_cast<bf16_t*>(dx), s));
  return DP_OK;
}


// ---- batched calls over the linear layers of one step ----
// The norm pass over all layers: with Hutch on bf16 inputs and every layer on
// the fused MFMA projection, one probe launch per kProbeLayersMax layers, the
// sketch and fused projection per layer into one row of partials per sample,
// and one per-sample sum; otherwise the per-layer calls one after another.
namespace {

struct LayersNormPlan {
  bool fused = false;
  size_t pb = 0, yb = 0, part = 0, total = 0;
  std::vector<int64_t> poff;   // per layer: first element of its probe block in pb
  std::vector<int> cols;       // per layer: column block of the fused projection
  std::vector<int64_t> pbase;  // per layer: first partial of its column blocks
  int64_t nparts = 0;          // partials per sample, all layers
};

bool layers_norm_ok(int method, int dtype, int B, int T, int k, int n, const dp_linear_layer_t* L) {
  if (n < 1 || L == nullptr) return false;
  for (int l = 0; l < n; ++l)
    if (!norm_args_ok(method, dtype, B, T, L[l].d, L[l].p, k)) return false;
  return true;
}

LayersNormPlan plan_norm_layers(int method, int dtype, int B, int T, int k, int n,
                                const dp_linear_layer_t* L) {
  LayersNormPlan P;
  bool fused = method == DP_NORM_HUTCH && dtype == DP_BF16 && k <= kMfmaProbeCols && B > 0 && T > 0;
  for (int l = 0; l < n && fused; ++l)
    fused = mfma_sketch_ok(T, L[l].p) && mfma_project_sq_cols(B, T, L[l].d) > 0;
  if (!fused) {
    for (int l = 0; l < n; ++l) {
      const size_t t = plan_norm(method, dtype, B, T, L[l].d, L[l].p, k).total;
      if (t > P.total) P.total = t;
    }
    return P;
  }
  P.fused = true;
  const size_t Bz = static_cast<size_t>(B);
  Carver pc;  // the probe blocks, one after another
  P.poff.resize(n);
  P.cols.resize(n);
  P.pbase.resize(n);
  for (int l = 0; l < n; ++l) {
    P.poff[l] = static_cast<int64_t>(pc.take(Bz * kMfmaProbeCols * L[l].p * 2) / 2);
    P.cols[l] = mfma_project_sq_cols(B, T, L[l].d);
    P.pbase[l] = P.nparts;
    P.nparts += L[l].d / P.cols[l];
  }
  Carver cv;
  P.pb = cv.take(pc.off);
  // one Y slab per layer of a launch group (kNormLayersMax layers per group)
  P.yb = cv.take(static_cast<size_t>(n < kNormLayersMax ? n : kNormLayersMax) * Bz * kMfmaProbeCols *
                 T * 2);
  P.part = cv.take(Bz * static_cast<size_t>(P.nparts) * sizeof(double));
  P.total = cv.off;
  return P;
}

// The batched update's contraction launches.  A layer on the MFMA contraction
// whose count of 256 x 256 output tiles is below 256 and divides it shares a
// launch with other layers of the same tile count, 256 / tiles of them (at
// most kGemmLayersMax), in the order of the call: a full group fills the chip
// without token splits, so its sums are written once, not as split planes that
// the update must add.  A layer left alone, and every other layer, takes the
// per-layer path.  Each unit's workspace is the clip prefix, then the unit's
// buffers (a group: every layer's planes, or its sum when unsplit).
struct UpdateUnit {
  int n = 0;
  bool grouped = false;
  int idx[kGemmLayersMax] = {};
  int tiles = 0;   // per layer (grouped units)
  int nsplit = 1;  // grouped units
  size_t buf[kGemmLayersMax] = {};
  size_t total = 0;
};
struct UpdateLayersPlan {
  std::vector<UpdateUnit> units;  // in the order of their first layer
  size_t total = 0;
};

UpdateLayersPlan plan_update_layers(int dtype, int B, int T, int n, const dp_linear_layer_t* L) {
  UpdateLayersPlan U;
  std::vector<int> open_unit(257, -1);  // the open group of each tile count
  for (int l = 0; l < n; ++l) {
    const AggPlan P = plan_agg(dtype, B, T, L[l].d, L[l].p, true);
    const int tiles = P.mfma ? mfma_gemm_tiles(L[l].d, L[l].p) : 0;
    if (tiles > 0 && tiles < 256 && 256 % tiles == 0) {
      const int cap = 256 / tiles < kGemmLayersMax ? 256 / tiles : kGemmLayersMax;
      int& u = open_unit[tiles];
      if (u < 0 || U.units[u].n == cap) {
        U.units.emplace_back();
        u = static_cast<int>(U.units.size()) - 1;
        U.units[u].grouped = true;
        U.units[u].tiles = tiles;
      }
      U.units[u].idx[U.units[u].n++] = l;
    } else {
      UpdateUnit one;
      one.n = 1;
      one.idx[0] = l;
      U.units.push_back(one);
    }
  }
  for (UpdateUnit& un : U.units) {
    if (un.grouped && un.n == 1) un.grouped = false;  // alone: the per-layer path
    if (!un.grouped) {
      const dp_linear_layer_t& ly = L[un.idx[0]];
      un.total = plan_agg(dtype, B, T, ly.d, ly.p, true).total;
    } else {
      un.nsplit = mfma_gemm_splits_tiles(B, T, static_cast<int64_t>(un.tiles) * un.n);
      Carver cv;
      AggPlan P;
      carve_agg_prefix(cv, P, B);
      for (int i = 0; i < un.n; ++i) {
        const dp_linear_layer_t& ly = L[un.idx[i]];
        un.buf[i] = cv.take(static_cast<size_t>(un.nsplit) * ly.p * ly.d * 4);
      }
      un.total = cv.off;
    }
    if (un.total > U.total) U.total = un.total;
  }
  return U;
}

}  // namespace

size_t dp_norm_est_layers_workspace(int method, int dtype, int B, int T, int k, int nlayers,
                                    const dp_linear_layer_t* layers) {
  if (!layers_norm_ok(method, dtype, B, T, k, nlayers, layers)) return kInvalid;
  return plan_norm_layers(method, dtype, B, T, k, nlayers, layers).total;
}

static dp_status_t norm_est_layers_impl(int method, int dtype, int B, int T, int k, int n,
                                        const dp_linear_layer_t* L, uint64_t seed,
                                        uint32_t flags, float* n_sq, void* ws, size_t ws_bytes,
                                        dp_stream_t stream, const Marks& mk) {
  if (!layers_norm_ok(method, dtype, B, T, k, n, L)) return DP_ERR_INVALID_ARG;
  if ((flags & ~(DP_ACCUMULATE | DP_PROBE_SHARED | DP_PROBE_RADEMACHER)) != 0)
    return DP_ERR_INVALID_ARG;
  if (B == 0) return DP_OK;
  if (n_sq == nullptr || !aligned(n_sq, 4)) return DP_ERR_INVALID_ARG;
  for (int l = 0; l < n; ++l)
    if (T > 0 && (L[l].A == nullptr || L[l].G == nullptr || !aligned(L[l].A, 16) ||
                  !aligned(L[l].G, 16)))
      return DP_ERR_INVALID_ARG;
  const LayersNormPlan P = plan_norm_layers(method, dtype, B, T, k, n, L);
  if (ws_bytes < P.total) return DP_ERR_WORKSPACE;
  if (P.total > 0 && (ws == nullptr || !aligned(ws, 16))) return DP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!P.fused) {  // the per-layer calls, accumulating after the first
    DP_TRY(mk.open(s));
    for (int l = 0; l < n; ++l) {
      const uint32_t f = l > 0 ? (flags | DP_ACCUMULATE) : flags;
      const dp_status_t st = norm_est_impl(method, dtype, B, T, L[l].d, L[l].p, k, L[l].A, L[l].G,
                                           seed, L[l].layer, f, n_sq, ws, ws_bytes, stream, Marks{});
      if (st != DP_OK) return st;
    }
    DP_TRY(mk.close(s));
    return DP_OK;
  }
  const bool shared = (flags & DP_PROBE_SHARED) != 0;
  const bool signs = (flags & DP_PROBE_RADEMACHER) != 0;
  const int nS = shared ? 1 : B;
  bf16_t* Pb = at<bf16_t>(ws, P.pb);
  bf16_t* Yb = at<bf16_t>(ws, P.yb);
  double* part = at<double>(ws, P.part);
  for (int c0 = 0; c0 < n; c0 += kProbeLayersMax) {
    ProbeLayerTable<kProbeLayersMax> tab{};
    tab.n = n - c0 < kProbeLayersMax ? n - c0 : kProbeLayersMax;
    int nb = 0;
    for (int t = 0; t < tab.n; ++t) {
      const dp_linear_layer_t& ly = L[c0 + t];
      tab.layer[t] = ly.layer;
      tab.p[t] = ly.p;
      tab.off[t] = P.poff[c0 + t];
      tab.bstart[t] = nb;
      nb += ((ly.p + 3) / 4 + 255) / 256;
    }
    tab.bstart[tab.n] = nb;
    DP_TRY(launch_probe_fill_layers_bf16(seed, tab, nS, k, kMfmaProbeCols, Pb, s, signs));
  }
  // Groups of up to kNormLayersMax layers: the sketches of a group, one launch per
  // sketch shape, then its projections, one launch per column block.
  const int64_t yslab = static_cast<int64_t>(B) * kMfmaProbeCols * T;  // elements
  DP_TRY(mk.open(s));
  for (int c0 = 0; c0 < n; c0 += kNormLayersMax) {
    const int cn = n - c0 < kNormLayersMax ? n - c0 : kNormLayersMax;
    for (int v = 0; v < 3; ++v) {
      SketchLayers tab{};
      for (int t = 0; t < cn; ++t) {
        const dp_linear_layer_t& ly = L[c0 + t];
        if (mfma_sketch_variant(B, T, ly.p) != v) continue;
        tab.X[tab.n] = static_cast<const bf16_t*>(ly.G);
        tab.P[tab.n] = Pb + P.poff[c0 + t];
        tab.Y[tab.n] = Yb + t * yslab;
        tab.W[tab.n] = ly.p;
        tab.pbs[tab.n] = shared ? 0 : static_cast<int64_t>(kMfmaProbeCols) * ly.p;
        ++tab.n;
      }
      if (tab.n > 0) DP_TRY(launch_sketch_mfma_layers(v, B, T, tab, s));
    }
    for (const int cols : {64, 128}) {
      ProjectLayers tab{};
      for (int t = 0; t < cn; ++t) {
        const dp_linear_layer_t& ly = L[c0 + t];
        if (P.cols[c0 + t] != cols) continue;
        tab.X[tab.n] = static_cast<const bf16_t*>(ly.A);
        tab.Y[tab.n] = Yb + t * yslab;
        tab.W[tab.n] = ly.d;
        tab.pbase[tab.n] = P.pbase[c0 + t];
        ++tab.n;
      }
      if (tab.n > 0)
        DP_TRY(launch_project_sq_mfma_layers(B, T, cols, tab, k, 1.0f / k, 0, 0.f, part, P.nparts,
                                             s));
    }
  }
  DP_TRY(mk.close(s));
  DP_TRY(launch_sum_parts(part, B, static_cast<int>(P.nparts), n_sq,
                          (flags & DP_ACCUMULATE) ? 1 : 0, s));
  return DP_OK;
}

dp_status_t dp_norm_est_layers(int method, int dtype, int B, int T, int k, int nlayers,
                               const dp_linear_layer_t* layers, uint64_t seed, uint32_t flags,
                               float* n_sq, void* ws, size_t ws_bytes, dp_stream_t stream) {
  return norm_est_layers_impl(method, dtype, B, T, k, nlayers, layers, seed, flags, n_sq, ws,
                              ws_bytes, stream, Marks{});
}

dp_status_t dp_norm_est_layers_timed(int method, int dtype, int B, int T, int k, int nlayers,
                                     const dp_linear_layer_t* layers, uint64_t seed,
                                     uint32_t flags, float* n_sq, void* ws, size_t ws_bytes,
                                     dp_stream_t stream, void* ev_begin, void* ev_end) {
  return norm_est_layers_impl(method, dtype, B, T, k, nlayers, layers, seed, flags, n_sq, ws,
                              ws_bytes, stream,
                              Marks{static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end)});
}

size_t dp_clip_aggregate_update_layers_workspace(int dtype, int B, int T, int nlayers,
                                                 const dp_linear_layer_t* layers) {
  if (nlayers < 1 || layers == nullptr) return kInvalid;
  for (int l = 0; l < nlayers; ++l)
    if (!agg_args_ok(dtype, B, T, layers[l].d, layers[l].p)) return kInvalid;
  return plan_update_layers(dtype, B, T, nlayers, layers).total;
}

int dp_clip_aggregate_update_layers_launches(int dtype, int B, int T, int nlayers,
                                             const dp_linear_layer_t* layers) {
  if (nlayers < 1 || layers == nullptr) return -1;
  for (int l = 0; l < nlayers; ++l)
    if (!agg_args_ok(dtype, B, T, layers[l].d, layers[l].p)) return -1;
  return static_cast<int>(plan_update_layers(dtype, B, T, nlayers, layers).units.size());
}

static dp_status_t update_layers_impl(int dtype, int B, int T, int n, const dp_linear_layer_t* L,
                                      const float* n_sq, float C, float sigma, float eta,
                                      uint64_t seed, float* c_out, void* ws, size_t ws_bytes,
                                      dp_stream_t stream, void* const* agg_begin,
                                      void* const* agg_end, void* const* upd_begin,
                                      void* const* upd_end) {
  if (n < 1 || L == nullptr) return DP_ERR_INVALID_ARG;
  for (int l = 0; l < n; ++l) {
    const dp_linear_layer_t& ly = L[l];
    if (!agg_args_ok(dtype, B, T, ly.d, ly.p)) return DP_ERR_INVALID_ARG;
    if (!update_args_ok(ly.d, ly.p, B, sigma, C, eta)) return DP_ERR_INVALID_ARG;
    if (!agg_ptrs_ok(B, T, ly.A, ly.G, n_sq, C, c_out)) return DP_ERR_INVALID_ARG;
    if (ly.theta == nullptr || !aligned(ly.theta, 16)) return DP_ERR_INVALID_ARG;
  }
  const UpdateLayersPlan U = plan_update_layers(dtype, B, T, n, L);
  const size_t need = U.total;
  if (ws_bytes < need) return DP_ERR_WORKSPACE;
  if (ws == nullptr || !aligned(ws, 16)) return DP_ERR_INVALID_ARG;
  for (int l = 0; l < n; ++l) {
    const size_t bytes = static_cast<size_t>(L[l].p) * L[l].d * 4;
    if (overlaps(L[l].theta, bytes, ws, need)) return DP_ERR_INVALID_ARG;
    for (int m = 0; m < l; ++m)
      if (overlaps(L[l].theta, bytes, L[m].theta, static_cast<size_t>(L[m].p) * L[m].d * 4))
        return DP_ERR_INVALID_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the clip factors once: the same n for every layer (the plans share the
  // status / c / order / count prefix, which depends on B only)
  const AggPlan P0 = plan_agg(dtype, B, T, L[0].d, L[0].p, true);
  DP_TRY(launch_clip(n_sq, B, C, at<float>(ws, P0.c), c_out, at<uint32_t>(ws, P0.status),
                     at<int>(ws, P0.order), at<int>(ws, P0.count), s));
  auto agg_marks = [&](int l) {
    return Marks{agg_begin ? static_cast<hipEvent_t>(agg_begin[l]) : nullptr,
                 agg_end ? static_cast<hipEvent_t>(agg_end[l]) : nullptr};
  };
  auto upd_marks = [&](int l) {
    return Marks{upd_begin ? static_cast<hipEvent_t>(upd_begin[l]) : nullptr,
                 upd_end ? static_cast<hipEvent_t>(upd_end[l]) : nullptr};
  };
  const float sigmaC = sigma * C;
  const float eta_over_B = static_cast<float>(static_cast<double>(eta) / B);
  for (const UpdateUnit& un : U.units) {
    if (!un.grouped) {
      const int l = un.idx[0];
      const dp_linear_layer_t& ly = L[l];
      const AggPlan P = plan_agg(dtype, B, T, ly.d, ly.p, true);
      const dp_status_t st = aggregate_update_layer(P, dtype, B, T, ly.d, ly.p, ly.A, ly.G, n_sq,
                                                    C, sigma, eta, seed, ly.layer, ly.theta,
                                                    nullptr, c_out, ws, s, agg_marks(l),
                                                    upd_marks(l), false);
      if (st != DP_OK) return st;
      continue;
    }
    GemmLayers tab;
    tab.n = un.n;
    int tiles = 0;
    for (int i = 0; i < un.n; ++i) {
      const dp_linear_layer_t& ly = L[un.idx[i]];
      tab.tile0[i] = tiles;
      tab.d[i] = ly.d;
      tab.p[i] = ly.p;
      tab.A[i] = static_cast<const bf16_t*>(ly.A);
      tab.G[i] = static_cast<const bf16_t*>(ly.G);
      tab.out[i] = at<float>(ws, un.buf[i]);
      tiles += un.tiles;
    }
    tab.tile0[un.n] = tiles;
    // the shared launch is timed in its first layer's pair; the others get an
    // empty pair right after it
    const Marks mk = agg_marks(un.idx[0]);
    DP_TRY(mk.open(s));
    DP_TRY(launch_aggregate_mfma_layers(B, T, tab, at<float>(ws, P0.c), at<int>(ws, P0.order),
                                        at<int>(ws, P0.count), un.nsplit, s));
    DP_TRY(mk.close(s));
    for (int i = 1; i < un.n; ++i) {
      const Marks mo = agg_marks(un.idx[i]);
      DP_TRY(mo.open(s));
      DP_TRY(mo.close(s));
    }
    for (int i = 0; i < un.n; ++i) {
      const dp_linear_layer_t& ly = L[un.idx[i]];
      const int64_t np = static_cast<int64_t>(ly.p) * ly.d;
      const Marks mu = upd_marks(un.idx[i]);
      DP_TRY(mu.open(s));
      if (un.nsplit == 1)
        DP_TRY(launch_noise_update(ly.theta, tab.out[i], np, sigmaC, eta_over_B, seed, ly.layer, s));
      else
        DP_TRY(launch_noise_update_splits(ly.theta, tab.out[i], un.nsplit, np, nullptr, sigmaC,
                                          eta_over_B, seed, ly.layer, s));
      DP_TRY(mu.close(s));
    }
  }
  return DP_OK;
}

dp_status_t dp_clip_aggregate_update_layers(int dtype, int B, int T, int nlayers,
                                            const dp_linear_layer_t* layers, const float* n_sq,
                                            float C, float sigma, float eta, uint64_t seed,
                                            float* c_out, void* ws, size_t ws_bytes,
                                            dp_stream_t stream) {
  return update_layers_impl(dtype, B, T, nlayers, layers, n_sq, C, sigma, eta, seed, c_out, ws,
                            ws_bytes, stream, nullptr, nullptr, nullptr, nullptr);
}

dp_status_t dp_clip_aggregate_update_layers_timed(int dtype, int B, int T, int nlayers,
                                                  const dp_linear_layer_t* layers,
                                                  const float* n_sq, float C, float sigma,
                                                  float eta, uint64_t seed, float* c_out,
                                                  void* ws, size_t ws_bytes, dp_stream_t stream,
                                                  void* const* agg_begin, void* const* agg_end,
                                                  void* const* upd_begin, void* const* upd_end) {
  return update_layers_impl(dtype, B, T, nlayers, layers, n_sq, C, sigma, eta, seed, c_out, ws,
                            ws_bytes, stream, agg_begin, agg_end, upd_begin, upd_end);
}


}  // extern "C"
