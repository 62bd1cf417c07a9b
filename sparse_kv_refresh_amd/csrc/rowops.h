// Row operations shared by the row kernels and the GEMM reductions that
// finish a residual row: one wavefront holds a row in registers, lane l owning
// elements l*4 + 256*j + 0..3 of chunk j, so every kernel that normalises a row
// this way sums in the same order and produces the same bits.
#pragma once

#include "common.h"

namespace wamc {

constexpr int kMaxRowChunks = 16;   // d <= 4096

// Chunks per lane that the row kernels hold in registers: the smallest of
// 1, 2, 4, 6, 8, 12, 16 covering d (fewer registers, more waves resident);
// 0 = d > 4096 (streaming).
inline int row_chunks(int d) {
  const int need = (d + 255) / 256;
  constexpr int kSizes[] = {1, 2, 4, 6, 8, 12, 16};
  for (int c : kSizes)
    if (need <= c) return c;
  return 0;
}

#define WAMC_ROW_NC_DISPATCH(nc, ...)                 \
  switch (nc) {                                       \
    case 1: { constexpr int NC = 1; __VA_ARGS__; } break;    \
    case 2: { constexpr int NC = 2; __VA_ARGS__; } break;    \
    case 4: { constexpr int NC = 4; __VA_ARGS__; } break;    \
    case 6: { constexpr int NC = 6; __VA_ARGS__; } break;    \
    case 8: { constexpr int NC = 8; __VA_ARGS__; } break;    \
    case 12: { constexpr int NC = 12; __VA_ARGS__; } break;  \
    case 16: { constexpr int NC = 16; __VA_ARGS__; } break;  \
    default: { constexpr int NC = 0; __VA_ARGS__; } break;   \
  }

// Row chunk j of a lane = elements lane*4 + 256*j + 0..3.  Every chunk load of
// a row is issued before the first use (one memory round trip per row); the
// chunk loop stops at the first chunk wholly past d (a uniform branch), lanes
// past d inside the last chunk re-read element 0 and are masked later.
template <int NC, typename T>
__device__ __forceinline__ void load_row(const T* __restrict__ p, int d, int lane, float (&v)[NC][4]) {
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    // chunks past d read column 0 (valid memory) and are never used; no
    // branch, so every load of the row is in flight at once
    const int c = lane * 4 + j * 256;
    const int cc = c < d ? c : 0;
    if constexpr (sizeof(T) == 2) {
      const uint2 raw = *reinterpret_cast<const uint2*>(p + cc);
      v[j][0] = __uint_as_float(raw.x << 16);
      v[j][1] = __uint_as_float(raw.x & 0xffff0000u);
      v[j][2] = __uint_as_float(raw.y << 16);
      v[j][3] = __uint_as_float(raw.y & 0xffff0000u);
    } else {
      const float4 f = *reinterpret_cast<const float4*>(p + cc);
      v[j][0] = f.x; v[j][1] = f.y; v[j][2] = f.z; v[j][3] = f.w;
    }
  }
}

// mean and 1/sqrt(var + eps) of a row held by one wavefront (biased variance,
// two passes over the registers; the summation order is fixed by the chunk
// assignment)
template <int NC>
__device__ __forceinline__ void row_stats(const float (&v)[NC][4], int d, int lane, float eps, float& mean,
                                          float& rstd) {
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (j * 256 >= d) break;
    if (lane * 4 + j * 256 < d) sum += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  }
  mean = wave_sum(sum) / static_cast<float>(d);
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (j * 256 >= d) break;
    if (lane * 4 + j * 256 < d) {
      const float a0 = v[j][0] - mean, a1 = v[j][1] - mean, a2 = v[j][2] - mean, a3 = v[j][3] - mean;
      q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float var = wave_sum(q) / static_cast<float>(d);
  rstd = 1.0f / sqrtf(var + eps);
}

// The shift/scale chunks of a row, loaded in the same batch as the row itself
// (they do not depend on it), so that one memory round trip covers both.
template <int NC, typename T, bool MOD>
struct RowMod {
  float sh[NC][4], sc[NC][4];
  __device__ __forceinline__ void load(const T* __restrict__ shift, const T* __restrict__ scale, int d, int lane) {
    if constexpr (MOD) {
      load_row<NC>(shift, d, lane, sh);
      load_row<NC>(scale, d, lane, sc);
    }
  }
};

// h = (v - mean) * rstd, times (1 + scale) plus shift when MOD, rounded to T
template <int NC, typename T, bool MOD>
__device__ __forceinline__ void row_norm_store(const float (&v)[NC][4], int d, int lane, float mean, float rstd,
                                               const RowMod<NC, T, MOD>& md, T* __restrict__ hr) {
  const auto& sh = md.sh;
  const auto& sc = md.sc;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (j * 256 >= d) break;
    const int c = lane * 4 + j * 256;
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float n = (v[j][i] - mean) * rstd;
      y[i] = MOD ? n * (1.0f + sc[j][i]) + sh[j][i] : n;
    }
    if (c < d) {
      if constexpr (sizeof(T) == 2) {
        uint2 w;
        w.x = pack_bf16x2(y[0], y[1]);
        w.y = pack_bf16x2(y[2], y[3]);
        *reinterpret_cast<uint2*>(hr + c) = w;
      } else {
        *reinterpret_cast<float4*>(hr + c) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
  }
}

}  // namespace wamc
