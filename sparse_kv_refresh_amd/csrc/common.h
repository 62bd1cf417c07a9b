// Device-side helpers shared by the libwamc kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wamc {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even, NaN stays NaN) in one
// v_cvt_pk_bf16_f32; lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.f) & 0xffffu);
}

// Element loads/stores for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Rows processed for episode b: k_eff[b] clamped to [0, cap], or cap when
// no count array is given (dense).
__device__ __forceinline__ int rows_of(const int32_t* k_eff, int b, int cap) {
  if (!k_eff) return cap;
  int k = k_eff[b];
  return k < 0 ? 0 : (k > cap ? cap : k);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Workgroup barrier that makes LDS writes visible but leaves vector-memory
// traffic (prefetches of the next tile) in flight; __syncthreads() would wait
// for those too.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));   // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
}

// Sum over the per-block surprise partials of one episode, by threads
// 0..255 of the calling block in a fixed order (so every kernel that needs
// sum_j U_j gets the same bits).  All threads of the block must call it.
__device__ __forceinline__ float usum_total(const float* __restrict__ usum_blocks, int nblocks, float* red4) {
  float acc = 0.f;
  if (threadIdx.x < 256)
    for (int i = threadIdx.x; i < nblocks; i += 256) acc += usum_blocks[i];
  acc = wave_sum(acc);
  if (threadIdx.x < 256 && (threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = acc;
  __syncthreads();
  return ((red4[0] + red4[1]) + red4[2]) + red4[3];
}

// score = w_a P / (L H A) + w_s U / sum(U)   (w_attn_norm = w_a / (L H A))
__device__ __forceinline__ float combine_score(float p, float u, float total, float w_attn_norm, float w_surprise) {
  float s = w_attn_norm * p;
  if (total > 0.f) s += w_surprise * (u / total);
  return s;
}

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8), each XCD
// with its own L2.  Remap a linear id so that XCD x receives the contiguous
// range [x*per, (x+1)*per) of work items (a bijection on [0, total)): work
// items that share operands then share an L2.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int kXcd = 8;
  const int per = (total + kXcd - 1) / kXcd;
  int tall = total % kXcd;
  if (tall == 0) tall = kXcd;
  const int xcd = pid % kXcd, local = pid / kXcd;
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// GELU with erf by the approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions (1964), formula 7.1.28: for u >= 0,
//   erf(u) = 1 - (1 + a1 u + a2 u^2 + ... + a6 u^6)^-16,  |error| <= 3e-7.
// Here u = |x| / sqrt(2), folded into the coefficients (c_i = a_i 2^(-i/2)),
// and with r = (1 + c1 |x| + ... + c6 |x|^6)^-16 = 1 - erf(|x|/sqrt(2)):
//   GELU(x) = x (1 + erf(x/sqrt2)) / 2 = max(x, 0) - |x| r / 2
// (for x < 0 the left side is x r / 2).  One reciprocal and no exponential;
// for large |x| the 16th power overflows to +inf and r to 0, which is the
// limit.  Used where the result is rounded to bf16 (relative precision
// 2^-8), so the approximation error does not show.
__device__ __forceinline__ float gelu_erf_fast(float x) {
  const float ax = fabsf(x);
  float q = fmaf(ax, 5.38297490e-06f, 4.88906371e-05f);
  q = fmaf(q, ax, 3.80035744e-05f);
  q = fmaf(q, ax, 3.27762635e-03f);
  q = fmaf(q, ax, 2.11410057e-02f);
  q = fmaf(q, ax, 4.98673469e-02f);
  q = fmaf(q, ax, 1.0f);
  q *= q;
  q *= q;
  q *= q;
  q *= q;
  const float r = __builtin_amdgcn_rcpf(q);
  return fmaf(-0.5f * ax, r, fmaxf(x, 0.0f));
}

}  // namespace wamc
