// Device helpers shared by the gfx950 kernels: bf16 storage, Philox4x32-10,
// Box-Muller, wave/block reductions.  HIP C++ for gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dprc {

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN) with gfx950's
// v_cvt_pk_bf16_f32: one instruction for a pair, no branch.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_hw v{static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.f) & 0xFFFFu);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ T to_out(float v);
template <> __device__ __forceinline__ float to_out<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t to_out<bf16_t>(float v) { return f32_to_bf16(v); }

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds on a 128-bit
// counter with a 64-bit key.  Each round takes the full 64-bit products of
// words 0 and 2 with the two round multipliers, and the key advances by the
// Weyl increments between rounds.
// ---------------------------------------------------------------------------
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;
constexpr uint32_t kNoiseC2 = 0xFFFFFFFFu;  // counter word 2 of the DP-noise stream

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one full 32 x 32 -> 64-bit product each (v_mad_u64_u32), not a low and a
    // high multiply
    const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c.z;
    const uint32_t lo0 = static_cast<uint32_t>(p0), hi0 = static_cast<uint32_t>(p0 >> 32);
    const uint32_t lo1 = static_cast<uint32_t>(p1), hi1 = static_cast<uint32_t>(p1 >> 32);
    u32x4 n;
    n.x = hi1 ^ c.y ^ k0;
    n.y = lo1;
    n.z = hi0 ^ c.w ^ k1;
    n.w = lo0;
    c = n;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return c;
}

// Two words -> two N(0,1) draws.  u1 = (top24(a) + 1) 2^-24 in (0, 1] and
// u2 = top24(b) 2^-24 in [0, 1) are exact in fp32; rho = sqrt(-2 ln u1) and the
// angle 2 pi u2 goes through sincospi(2 u2) (no rounding of pi).
__device__ __forceinline__ void box_muller(uint32_t a, uint32_t b, float& z0, float& z1) {
  const float u1 = static_cast<float>((a >> 8) + 1u) * 0x1p-24f;
  const float u2 = static_cast<float>(b >> 8) * 0x1p-24f;
  const float rho = sqrtf(-2.0f * logf(u1));
  float s, c;
  sincospif(2.0f * u2, &s, &c);
  z0 = rho * c;
  z1 = rho * s;
}

// Counter of the DP-noise stream for the group of four flat parameter indices
// 4 grp .. 4 grp + 3 of `layer`: (lo(grp), hi(grp), 0xFFFFFFFF, layer).
__device__ __forceinline__ u32x4 noise_counter(uint64_t grp, uint32_t layer) {
  u32x4 c;
  c.x = static_cast<uint32_t>(grp);
  c.y = static_cast<uint32_t>(grp >> 32);
  c.z = kNoiseC2;
  c.w = layer;
  return c;
}

__device__ __forceinline__ void normals4(u32x4 ctr, uint32_t k0, uint32_t k1, float z[4]) {
  const u32x4 w = philox4x32_10(ctr, k0, k1);
  box_muller(w.x, w.y, z[0], z[1]);
  box_muller(w.z, w.w, z[2], z[3]);
}

// ---------------------------------------------------------------------------
// Deterministic reductions (fixed order for a fixed launch shape).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Block sum for blockDim.x a multiple of 64 and <= 1024; result valid in all threads.
__device__ __forceinline__ float block_sum(float v, float* red /* >= 16 floats LDS */) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

__device__ __forceinline__ double block_sum_d(double v, double* red /* >= 16 doubles LDS */) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum_d(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

}  // namespace dprc
