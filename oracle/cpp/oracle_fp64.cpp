// Plain C++17 fp64 CPU oracle of the DP-SGD-RC hot path (Hutch norms, clip
// factors, clipped sum, Gaussian noise and SGD update).
//
// TEST INFRASTRUCTURE ONLY: called from tests/ and from bench.py's CPU
// baseline through oracle/cpp_oracle.py; nothing in the product path loads
// it.  It shares no code with the GPU library.  No BLAS: every product is a
// plain loop nest (blocked for the cache), threads are std::thread.
//
// Sources, by the titles and sections of the pages:
//  - randomized-clipping summary ("技術的サマリー：ランダム化クリッピングを備えた
//    LLM 向け効率的な DP-SGD"), section 中核メカニズム, item 1: the Hutchinson
//    estimate of tr(G^T A A^T G) = ||A^T G||_F^2 with a Gaussian p x k probe,
//    computed as ||A^T (G P)||_F^2 / k (the 1/k makes N(0, 1) probes
//    unbiased); section アルゴリズム的フロー, steps 3-5;
//  - DP-SGD glossary ("DP-SGD（差分プライバシー確率的勾配降下法）とは？"),
//    section DP-SGDのアルゴリズム, steps 3-5: c_i = min(1, C / ||g_i||), the
//    clipped sum, noise N(0, sigma^2 C^2 I) and theta <- theta - (eta / |B|) (.).
//  - Philox4x32-10 from its published definition (Salmon, Moraes, Dror and
//    Shaw, SC'11); Box-Muller from its mathematics.  The bit streams (24-bit
//    uniforms, lanes, counter words) are the readings the numpy oracle states.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---- Philox4x32-10 ----
struct U4 {
  uint32_t v[4];
};

U4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint64_t seed) {
  uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  uint32_t x0 = c0, x1 = c1, x2 = c2, x3 = c3;
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {  // the key is bumped by the Weyl constants between rounds
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * x0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * x2;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
  }
  return U4{{x0, x1, x2, x3}};
}

// Four words -> four N(0, 1): words (0, 1) and (2, 3) each give a Box-Muller
// pair from 24-bit uniforms u1 = (m + 1) 2^-24 in (0, 1], u2 = m 2^-24.
void box_muller4(const U4& w, double z[4]) {
  for (int a = 0; a < 4; a += 2) {
    const double u1 = (static_cast<double>(w.v[a] >> 8) + 1.0) * 0x1p-24;
    const double u2 = static_cast<double>(w.v[a + 1] >> 8) * 0x1p-24;
    const double rho = std::sqrt(-2.0 * std::log(u1));
    const double ang = 2.0 * M_PI * u2;
    z[a] = rho * std::cos(ang);
    z[a + 1] = rho * std::sin(ang);
  }
}

// ---- inputs: the bytes the GPU reads, upcast exactly ----
double elem(int dtype, const void* base, int64_t i) {
  if (dtype == 1) {  // bfloat16: the top half of an fp32
    uint16_t h;
    std::memcpy(&h, static_cast<const unsigned char*>(base) + 2 * i, 2);
    const uint32_t bits = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &bits, 4);
    return f;
  }
  float f;
  std::memcpy(&f, static_cast<const unsigned char*>(base) + 4 * i, 4);
  return f;
}

int threads_or_default(int n) {
  if (n > 0) return n;
  const unsigned h = std::thread::hardware_concurrency();
  return h > 0 ? static_cast<int>(h) : 1;
}

// Run f(lo, hi) over [0, n) split into nthreads contiguous ranges.
template <typename F>
void parallel_for(int64_t n, int nthreads, F f) {
  const int nt = static_cast<int>(std::min<int64_t>(nthreads, n > 0 ? n : 1));
  std::vector<std::thread> ts;
  for (int t = 0; t < nt; ++t) {
    const int64_t lo = n * t / nt, hi = n * (t + 1) / nt;
    ts.emplace_back([=] { f(lo, hi); });
  }
  for (auto& t : ts) t.join();
}

// The probe of (seed, layer, sample): P[r][j] is lane r mod 4 of the Philox
// counter (r / 4, j, sample, layer).
void probe(uint64_t seed, uint32_t layer, uint32_t sample, int p, int k, double* P) {
  for (int g = 0; 4 * g < p; ++g)
    for (int j = 0; j < k; ++j) {
      double z[4];
      box_muller4(philox(static_cast<uint32_t>(g), static_cast<uint32_t>(j), sample, layer, seed),
                  z);
      for (int l = 0; l < 4 && 4 * g + l < p; ++l) P[static_cast<int64_t>(4 * g + l) * k + j] = z[l];
    }
}

}  // namespace

extern "C" {

int oc_hardware_concurrency(void) { return threads_or_default(0); }

// out[4 i .. 4 i + 3] = Philox4x32-10 of counter ctr[4 i .. 4 i + 3] under `seed`.
void oc_philox(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    const U4 w = philox(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3], seed);
    for (int l = 0; l < 4; ++l) out[4 * i + l] = w.v[l];
  }
}

// P [p][k] of (seed, layer, sample), fp64.
void oc_probe(uint64_t seed, uint32_t layer, uint32_t sample, int p, int k, double* P) {
  probe(seed, layer, sample, p, k, P);
}

// Hutch squared norms of one layer for every sample: n[i] = ||A_i^T (G_i P_i)||_F^2 / k
// (or n[i] += with accumulate).  A [B][T][d], G [B][T][p] of `dtype` (0 fp32, 1 bf16).
void oc_hutch_norms(int dtype, int B, int T, int d, int p, int k, const void* A, const void* G,
                    uint64_t seed, uint32_t layer, int accumulate, int nthreads, double* n) {
  nthreads = threads_or_default(nthreads);
  std::vector<double> P(static_cast<size_t>(p) * k), Y(static_cast<size_t>(T) * k),
      Z(static_cast<size_t>(d) * k);
  for (int i = 0; i < B; ++i) {
    probe(seed, layer, static_cast<uint32_t>(i), p, k, P.data());
    const int64_t a0 = static_cast<int64_t>(i) * T * d, g0 = static_cast<int64_t>(i) * T * p;
    // Y = G_i P  (T x k), rows split over the threads
    parallel_for(T, nthreads, [&](int64_t lo, int64_t hi) {
      for (int64_t t = lo; t < hi; ++t) {
        double* y = &Y[t * k];
        for (int j = 0; j < k; ++j) y[j] = 0.0;
        for (int r = 0; r < p; ++r) {
          const double gv = elem(dtype, G, g0 + t * p + r);
          const double* pr = &P[static_cast<int64_t>(r) * k];
          for (int j = 0; j < k; ++j) y[j] += gv * pr[j];
        }
      }
    });
    // Z = A_i^T Y  (d x k), rows of Z split over the threads
    parallel_for(d, nthreads, [&](int64_t lo, int64_t hi) {
      for (int64_t q = lo; q < hi; ++q)
        for (int j = 0; j < k; ++j) Z[q * k + j] = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        const double* y = &Y[t * k];
        for (int64_t q = lo; q < hi; ++q) {
          const double av = elem(dtype, A, a0 + t * d + q);
          double* z = &Z[q * k];
          for (int j = 0; j < k; ++j) z[j] += av * y[j];
        }
      }
    });
    double s = 0.0;
    for (size_t e = 0; e < Z.size(); ++e) s += Z[e] * Z[e];
    s /= k;
    n[i] = accumulate ? n[i] + s : s;
  }
}

// c[i] = 1 if n[i] <= C^2, C / sqrt(n[i]) above, 0 (and the returned flag) if n[i]
// is not finite.
int oc_clip(int B, const double* n, double C, double* c) {
  int flag = 0;
  for (int i = 0; i < B; ++i) {
    if (!std::isfinite(n[i])) {
      c[i] = 0.0;
      flag = 1;
    } else if (n[i] <= C * C) {
      c[i] = 1.0;
    } else {
      c[i] = C / std::sqrt(n[i]);
    }
  }
  return flag;
}

// S[o][q] = sum_i c_i sum_t G_i[t][o] A_i[t][q]  ((p, d) layout), blocked over
// (o, q) tiles that the threads take in turn.
void oc_aggregate(int dtype, int B, int T, int d, int p, const void* A, const void* G,
                  const double* c, int nthreads, double* S) {
  nthreads = threads_or_default(nthreads);
  constexpr int kO = 32, kQ = 256;
  const int64_t to = (p + kO - 1) / kO, tq = (d + kQ - 1) / kQ;
  parallel_for(to * tq, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<double> acc(static_cast<size_t>(kO) * kQ), a(kQ), g(kO);
    for (int64_t tile = lo; tile < hi; ++tile) {
      const int o0 = static_cast<int>(tile / tq) * kO, q0 = static_cast<int>(tile % tq) * kQ;
      const int no = std::min(kO, p - o0), nq = std::min(kQ, d - q0);
      std::fill(acc.begin(), acc.end(), 0.0);
      for (int i = 0; i < B; ++i) {
        if (c[i] == 0.0) continue;
        const int64_t a0 = static_cast<int64_t>(i) * T * d, g0 = static_cast<int64_t>(i) * T * p;
        for (int t = 0; t < T; ++t) {
          for (int q = 0; q < nq; ++q) a[q] = elem(dtype, A, a0 + static_cast<int64_t>(t) * d + q0 + q);
          for (int o = 0; o < no; ++o)
            g[o] = c[i] * elem(dtype, G, g0 + static_cast<int64_t>(t) * p + o0 + o);
          for (int o = 0; o < no; ++o) {
            double* row = &acc[static_cast<size_t>(o) * kQ];
            const double go = g[o];
            for (int q = 0; q < nq; ++q) row[q] += go * a[q];
          }
        }
      }
      for (int o = 0; o < no; ++o)
        for (int q = 0; q < nq; ++q)
          S[static_cast<int64_t>(o0 + o) * d + q0 + q] = acc[static_cast<size_t>(o) * kQ + q];
    }
  });
}

// theta[e] -= (eta / B) (S[e] + sigma C xi[e]) for the n elements e in
// [offset, offset + n) of a (p, d) parameter (theta and S hold those n
// elements); xi[e] is lane e mod 4 of the counter (lo(e / 4), hi(e / 4),
// 0xFFFFFFFF, layer).
void oc_noise_update(int64_t offset, int64_t n, double* theta, const double* S, double sigma,
                     double C, double eta, int B, uint64_t seed, uint32_t layer, int nthreads) {
  nthreads = threads_or_default(nthreads);
  const double step = eta / B;
  parallel_for(n, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t idx = lo; idx < hi; ++idx) {
      const uint64_t e = static_cast<uint64_t>(offset + idx), grp = e >> 2;
      double z[4];
      box_muller4(philox(static_cast<uint32_t>(grp), static_cast<uint32_t>(grp >> 32),
                         0xFFFFFFFFu, layer, seed),
                  z);
      theta[idx] -= step * (S[idx] + sigma * C * z[e & 3]);
    }
  });
}

}  // extern "C"
