// Row kernels: gather of the refreshed rows (with the reference-embedding
// update) and the modulated LayerNorm that feeds each projection.
//
// WAM-Cache (paperpeel 2610.11401) §4.1: the reference embedding of a token is
// its input embedding at the most recent refresh, so zref is overwritten for
// exactly the refreshed tokens; §3: each DiT sub-layer starts from a
// (modulated) normalisation of its input.
//
// Both kernels give one wavefront per row and move 16-byte vectors so a row
// of d elements is read and written with fully coalesced accesses.
#include "common.h"
#include "launch.h"
#include "rowops.h"

namespace wamc {

constexpr int kRowThreads = 256;   // 4 rows per block

// every block zeroes its grid-strided share of the side job's arrays
__device__ __forceinline__ void zero_job(const ZeroJob& zj) {
  const int nthreads = gridDim.x * gridDim.y * kRowThreads;
  const int i0 = (blockIdx.y * gridDim.x + blockIdx.x) * kRowThreads + threadIdx.x;
  for (int i = i0; i < zj.n0; i += nthreads) zj.p0[i] = 0;
  for (int i = i0; i < zj.n1; i += nthreads) zj.p1[i] = 0;
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void gather_kernel(
    const T* __restrict__ z, T* __restrict__ zref, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ k_eff, int N, int d, int rows_cap, float* __restrict__ x,
    int32_t* __restrict__ age_zero, ZeroJob zj) {
  zero_job(zj);
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = blockIdx.x * (kRowThreads / kWave) + wid;
  if (r >= rows_of(k_eff, b, rows_cap)) return;
  const int t = idx ? idx[static_cast<size_t>(b) * N + r] : r;
  if (t < 0 || t >= N) return;
  const size_t src = (static_cast<size_t>(b) * N + t) * d;
  float* xr = x + (static_cast<size_t>(b) * rows_cap + r) * d;
  // 16-byte chunks lane*8 + 512*j, four in flight at a time
  constexpr int kPer = 16 / sizeof(T);   // elements per 16-byte load
  for (int c0 = lane * 8; c0 < d; c0 += 4 * kWave * 8) {
    uint4 raw[4][8 / kPer];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + q * kWave * 8 < d ? c0 + q * kWave * 8 : c0;
#pragma unroll
      for (int u = 0; u < 8 / kPer; ++u) raw[q][u] = *reinterpret_cast<const uint4*>(z + src + c + u * kPer);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + q * kWave * 8;
      if (c >= d) continue;
      float4 lo, hi;
      if constexpr (sizeof(T) == 2) {
        const uint32_t w[4] = {raw[q][0].x, raw[q][0].y, raw[q][0].z, raw[q][0].w};
        lo.x = __uint_as_float(w[0] << 16); lo.y = __uint_as_float(w[0] & 0xffff0000u);
        lo.z = __uint_as_float(w[1] << 16); lo.w = __uint_as_float(w[1] & 0xffff0000u);
        hi.x = __uint_as_float(w[2] << 16); hi.y = __uint_as_float(w[2] & 0xffff0000u);
        hi.z = __uint_as_float(w[3] << 16); hi.w = __uint_as_float(w[3] & 0xffff0000u);
      } else {
        lo = __builtin_bit_cast(float4, raw[q][0]);
        hi = __builtin_bit_cast(float4, raw[q][8 / kPer - 1]);
      }
      *reinterpret_cast<float4*>(xr + c) = lo;
      *reinterpret_cast<float4*>(xr + c + 4) = hi;
      if (zref) {
#pragma unroll
        for (int u = 0; u < 8 / kPer; ++u) *reinterpret_cast<uint4*>(zref + src + c + u * kPer) = raw[q][u];
      }
    }
  }
  if (age_zero && lane == 0) age_zero[static_cast<size_t>(b) * N + t] = 0;
}

hipError_t launch_gather(bool bf16, const void* z, void* zref, const int32_t* idx, const int32_t* k_eff,
                         int B, int N, int d, int rows_cap, float* x, int32_t* age_zero, const ZeroJob& zj,
                         hipStream_t s, KernelTimer* timer) {
  TimedLaunch t(timer, "gather", s);
  const dim3 grid((rows_cap + 3) / 4, B);
  if (bf16)
    launch(gather_kernel<bf16_t>, grid, kRowThreads, 0, s, static_cast<const bf16_t*>(z),
        static_cast<bf16_t*>(zref), idx, k_eff, N, d, rows_cap, x, age_zero, zj);
  else
    launch(gather_kernel<float>, grid, kRowThreads, 0, s, static_cast<const float*>(z),
        static_cast<float*>(zref), idx, k_eff, N, d, rows_cap, x, age_zero, zj);
  return hipGetLastError();
}

// Gather fused with the first modulated LayerNorm of layer 0: the row is
// held in registers, x and zref are written, and h = LN(x)(1+scale)+shift is
// produced in the same pass.  Each lane owns elements lane*4 + 256*j + 0..3,
// the assignment (and so the summation order) of the stand-alone LayerNorm
// kernel below, so both give the same bits.
template <int NC, typename T>
__global__ __launch_bounds__(kRowThreads) void gather_ln_kernel(
    const T* __restrict__ z, T* __restrict__ zref, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ k_eff, int N, int d, int rows_cap, float* __restrict__ x,
    int32_t* __restrict__ age_zero, const T* __restrict__ shift, const T* __restrict__ scale, float eps,
    T* __restrict__ h, ZeroJob zj) {
  zero_job(zj);
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = blockIdx.x * (kRowThreads / kWave) + wid;
  if (r >= rows_of(k_eff, b, rows_cap)) return;
  const int t = idx ? idx[static_cast<size_t>(b) * N + r] : r;
  if (t < 0 || t >= N) return;
  const size_t src = (static_cast<size_t>(b) * N + t) * d;
  const size_t row = static_cast<size_t>(b) * rows_cap + r;
  float* xr = x + row * d;
  float v[NC][4];
  load_row<NC>(z + src, d, lane, v);
  RowMod<NC, T, true> md;
  md.load(shift, scale, d, lane);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (j * 256 >= d) break;
    const int c = lane * 4 + j * 256;
    if (c < d) {
      if constexpr (sizeof(T) == 2) {
        // the values are bf16, so their upper halves are the original bits
        uint2 raw;
        raw.x = (__float_as_uint(v[j][0]) >> 16) | (__float_as_uint(v[j][1]) & 0xffff0000u);
        raw.y = (__float_as_uint(v[j][2]) >> 16) | (__float_as_uint(v[j][3]) & 0xffff0000u);
        *reinterpret_cast<uint2*>(zref + src + c) = raw;
      } else {
        *reinterpret_cast<float4*>(zref + src + c) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
      }
      *reinterpret_cast<float4*>(xr + c) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
    }
  }
  if (age_zero && lane == 0) age_zero[static_cast<size_t>(b) * N + t] = 0;
  float mean, rstd;
  row_stats(v, d, lane, eps, mean, rstd);
  row_norm_store<NC, T, true>(v, d, lane, mean, rstd, md, h + row * d);
}

hipError_t launch_gather_ln(bool bf16, const void* z, void* zref, const int32_t* idx, const int32_t* k_eff, int B,
                            int N, int d, int rows_cap, float* x, int32_t* age_zero, const void* shift,
                            const void* scale, float eps, void* h, const ZeroJob& zj, hipStream_t s,
                            KernelTimer* timer) {
  if (d > kMaxRowChunks * 256) return hipErrorInvalidValue;
  TimedLaunch t(timer, "gather_ln", s);
  const dim3 grid((rows_cap + 3) / 4, B);
  const int nc = row_chunks(d);
  if (bf16) {
    WAMC_ROW_NC_DISPATCH(nc, if constexpr (NC > 0) launch(gather_ln_kernel<NC, bf16_t>, grid, kRowThreads, 0, s,
        static_cast<const bf16_t*>(z), static_cast<bf16_t*>(zref), idx, k_eff, N, d, rows_cap, x, age_zero,
        static_cast<const bf16_t*>(shift), static_cast<const bf16_t*>(scale), eps, static_cast<bf16_t*>(h), zj))
  } else {
    WAMC_ROW_NC_DISPATCH(nc, if constexpr (NC > 0) launch(gather_ln_kernel<NC, float>, grid, kRowThreads, 0, s,
        static_cast<const float*>(z), static_cast<float*>(zref), idx, k_eff, N, d, rows_cap, x, age_zero,
        static_cast<const float*>(shift), static_cast<const float*>(scale), eps, static_cast<float*>(h), zj))
  }
  return hipGetLastError();
}

// LayerNorm without affine (biased variance), then *(1 + scale) + shift
// (MOD; without: the plain normalisation, as the cross-attention queries
// use), rounded to the activation type.
template <int NC, typename T, bool MOD>
__global__ __launch_bounds__(kRowThreads) void ln_mod_kernel(
    const float* __restrict__ x, const T* __restrict__ shift, const T* __restrict__ scale,
    int rows_cap, const int32_t* __restrict__ k_eff, int d, float eps, T* __restrict__ h, ZeroJob zj) {
  zero_job(zj);
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = blockIdx.x * (kRowThreads / kWave) + wid;
  if (r >= rows_of(k_eff, b, rows_cap)) return;
  const size_t row = static_cast<size_t>(b) * rows_cap + r;
  if constexpr (NC > 0) {
    float v[NC][4];
    load_row<NC>(x + row * d, d, lane, v);
    RowMod<NC, T, MOD> md;
    md.load(shift, scale, d, lane);
    float mean, rstd;
    row_stats(v, d, lane, eps, mean, rstd);
    row_norm_store<NC, T, MOD>(v, d, lane, mean, rstd, md, h + row * d);
  } else {
    // rows too long for registers: three streaming passes, same chunk
    // assignment and summation order
    const float* xr = x + row * d;
    T* hr = h + row * d;
    float s = 0.f;
    for (int c = lane * 4; c < d; c += kWave * 4) {
      const float4 v = *reinterpret_cast<const float4*>(xr + c);
      s += (v.x + v.y) + (v.z + v.w);
    }
    const float mean = wave_sum(s) / static_cast<float>(d);
    float q = 0.f;
    for (int c = lane * 4; c < d; c += kWave * 4) {
      const float4 v = *reinterpret_cast<const float4*>(xr + c);
      const float a = v.x - mean, bb = v.y - mean, cc = v.z - mean, dd = v.w - mean;
      q += (a * a + bb * bb) + (cc * cc + dd * dd);
    }
    const float var = wave_sum(q) / static_cast<float>(d);
    const float rstd = 1.0f / sqrtf(var + eps);
    for (int c = lane * 4; c < d; c += kWave * 4) {
      const float4 v = *reinterpret_cast<const float4*>(xr + c);
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float n = (vv[i] - mean) * rstd;
        const float y = MOD ? n * (1.0f + Elem<T>::load(scale, c + i)) + Elem<T>::load(shift, c + i) : n;
        Elem<T>::store(hr, c + i, y);
      }
    }
  }
}

hipError_t launch_ln_mod(bool bf16, const float* x, const void* shift, const void* scale, int B,
                         int rows_cap, const int32_t* k_eff, int d, float eps, void* h, const ZeroJob& zj,
                         hipStream_t s, KernelTimer* timer) {
  TimedLaunch t(timer, "ln_mod", s);
  const dim3 grid((rows_cap + 3) / 4, B);
  const bool mod = shift != nullptr;
  const int nc = row_chunks(d);
  if (bf16 && mod) {
    WAMC_ROW_NC_DISPATCH(nc, launch(ln_mod_kernel<NC, bf16_t, true>, grid, kRowThreads, 0, s, x,
        static_cast<const bf16_t*>(shift), static_cast<const bf16_t*>(scale), rows_cap, k_eff, d, eps,
        static_cast<bf16_t*>(h), zj))
  } else if (bf16) {
    WAMC_ROW_NC_DISPATCH(nc, launch(ln_mod_kernel<NC, bf16_t, false>, grid, kRowThreads, 0, s, x, nullptr, nullptr,
        rows_cap, k_eff, d, eps, static_cast<bf16_t*>(h), zj))
  } else if (mod) {
    WAMC_ROW_NC_DISPATCH(nc, launch(ln_mod_kernel<NC, float, true>, grid, kRowThreads, 0, s, x,
        static_cast<const float*>(shift), static_cast<const float*>(scale), rows_cap, k_eff, d, eps,
        static_cast<float*>(h), zj))
  } else {
    WAMC_ROW_NC_DISPATCH(nc, launch(ln_mod_kernel<NC, float, false>, grid, kRowThreads, 0, s, x, nullptr, nullptr,
        rows_cap, k_eff, d, eps, static_cast<float*>(h), zj))
  }
  return hipGetLastError();
}

}  // namespace wamc
