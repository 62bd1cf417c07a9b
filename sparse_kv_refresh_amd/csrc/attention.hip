// Attention of the refreshed queries over all N cached keys.
//
// WAM-Cache (paperpeel 2610.11401) §3: each query attends over all S_v keys
// and values; §4.4: a refreshed query attends over retained K/V of
// unrefreshed tokens and the fresh K/V of refreshed ones (the QKV epilogue
// has already written the fresh rows into the cache).  Non-causal, no mask.
//
// bf16 path (head_dim 128): flash-style, one workgroup per (128-query tile,
// head, episode), 4 waves x 32 queries, keys streamed through LDS 64 at a
// time with an online softmax (log2 domain, f32).
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K is the A operand (read from
//     LDS), Q^T the B operand (held in registers for the whole sweep).  The
//     result layout gives each lane one query and 32 of the tile's keys, so
//     the row max / row sum need one cross-half exchange only.
//   * O^T += V^T P^T on the same MFMA: P^T is taken straight from the S^T
//     accumulator registers (converted to bf16), V^T comes from a transposed
//     copy of the V tile in LDS; each A fragment is two 8-byte LDS reads.
//   * The next tile's K/V rows are fetched into registers while the current
//     tile is multiplied (single LDS buffer, two barriers per tile).
// fp32 path: one wavefront per query row with a VALU online softmax.
#include "common.h"
#include "launch.h"

namespace wamc {

constexpr float kLog2e = 1.4426950408889634f;

constexpr int kAttnThreads = 256;
constexpr int kAttnQ = 128;            // queries per workgroup
constexpr int kAttnKeys = 64;          // keys per tile
constexpr int kDh = 128;
constexpr int kKsStride = kDh + 8;     // padded LDS rows (bf16)
constexpr int kVtStride = kAttnKeys + 4;

__global__ __launch_bounds__(kAttnThreads, 2) void attn_bf16_kernel(AttnArgs a, float scale2) {
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int rows = rows_of(a.k_eff, b, a.rows_cap);
  const int q0 = qt * kAttnQ;
  if (q0 >= rows) return;

  __shared__ bf16_t Ks[kAttnKeys * kKsStride];
  __shared__ bf16_t Vt[kDh * kVtStride];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int N = a.N, d = a.d;
  const bf16_t* Kc = static_cast<const bf16_t*>(a.k_cache) + static_cast<size_t>(b) * N * d + h * kDh;
  const bf16_t* Vc = static_cast<const bf16_t*>(a.v_cache) + static_cast<size_t>(b) * N * d + h * kDh;

  // Q^T fragments: lane (half, col) = query q0 + wid*32 + col,
  // k-step s slot j <-> dh = s*16 + half*8 + j
  const int qrow = q0 + wid * 32 + col;
  const bf16_t* Qp = static_cast<const bf16_t*>(a.q) + (static_cast<size_t>(b) * a.rows_cap + qrow) * d + h * kDh;
  uint4 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = qrow < rows ? *reinterpret_cast<const uint4*>(Qp + s * 16 + half * 8) : make_uint4(0, 0, 0, 0);

  uint4 rk[4], rv[4];
  auto load_tile = [&](int kbase) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = tid + i * kAttnThreads;
      const int kk = kbase + (chunk >> 4), c8 = (chunk & 15) * 8;          // K: 16 threads per row
      rk[i] = kk < N ? *reinterpret_cast<const uint4*>(Kc + static_cast<size_t>(kk) * d + c8)
                     : make_uint4(0, 0, 0, 0);
      const int kv = kbase + (chunk & 63), c8v = (chunk >> 6) * 8;        // V: a wave spans 64 keys
      rv[i] = kv < N ? *reinterpret_cast<const uint4*>(Vc + static_cast<size_t>(kv) * d + c8v)
                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = tid + i * kAttnThreads;
      *reinterpret_cast<uint4*>(&Ks[(chunk >> 4) * kKsStride + (chunk & 15) * 8]) = rk[i];
      const int kv = chunk & 63, c8v = (chunk >> 6) * 8;
      const uint32_t w[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Vt[(c8v + 2 * j) * kVtStride + kv] = static_cast<bf16_t>(w[j] & 0xffffu);
        Vt[(c8v + 2 * j + 1) * kVtStride + kv] = static_cast<bf16_t>(w[j] >> 16);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_t{};

  const int ntiles = (N + kAttnKeys - 1) / kAttnKeys;
  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile((t + 1) * kAttnKeys);

    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16_t* kr = &Ks[(kb * 32 + col) * kKsStride + half * 8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kr + s * 16));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, __builtin_bit_cast(bf16x8_t, qf[s]), sacc[kb], 0, 0, 0);
      }
    }
    // sacc[kb][v]: key t*64 + kb*32 + (v/4)*8 + half*4 + v%4, query col
    const int kbase = t * kAttnKeys;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kbase + kb * 32 + (v / 4) * 8 + half * 4 + (v % 4);
        const float sv = key < N ? sacc[kb][v] * scale2 : -INFINITY;
        sacc[kb][v] = sv;
        tmax = fmaxf(tmax, sv);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2f(sacc[kb][v] - m_new);
        sacc[kb][v] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;

    // O^T[dh][q] += V^T[dh][key] P^T[key][q]; step (kb, tt) covers keys
    // kb*32 + 16*tt + (j/4)*8 + half*4 + j%4 for slot j
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint4 pk;
        pk.x = pack_bf16x2(sacc[kb][8 * tt + 0], sacc[kb][8 * tt + 1]);
        pk.y = pack_bf16x2(sacc[kb][8 * tt + 2], sacc[kb][8 * tt + 3]);
        pk.z = pack_bf16x2(sacc[kb][8 * tt + 4], sacc[kb][8 * tt + 5]);
        pk.w = pack_bf16x2(sacc[kb][8 * tt + 6], sacc[kb][8 * tt + 7]);
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pk);
        const int koff = kb * 32 + 16 * tt + half * 4;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16_t* vr = &Vt[(db * 32 + col) * kVtStride + koff];
          const uint2 lo = *reinterpret_cast<const uint2*>(vr);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
        }
      }
  }

  const float l = l_run + __shfl_xor(l_run, 32, kWave);
  if (qrow >= rows) return;
  const float inv = 1.0f / l;
  bf16_t* Op = static_cast<bf16_t*>(a.o) + (static_cast<size_t>(b) * a.rows_cap + qrow) * d + h * kDh;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      // elements v = g4*4 .. g4*4+3: dh rows db*32 + g4*8 + half*4 + 0..3
      uint2 w;
      w.x = pack_bf16x2(o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv);
      w.y = pack_bf16x2(o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(Op + db * 32 + g4 * 8 + half * 4) = w;
    }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------

constexpr int kF32MaxDh = 128;

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a, float scale2) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int rows = rows_of(a.k_eff, b, a.rows_cap);
  const int r = blockIdx.x * 4 + wid;
  __shared__ float sq[4][kF32MaxDh];
  const int N = a.N, d = a.d, dh = a.dh;
  if (r >= rows) return;
  const float* Q = static_cast<const float*>(a.q) + (static_cast<size_t>(b) * a.rows_cap + r) * d + h * dh;
  for (int c = lane; c < dh; c += kWave) sq[wid][c] = Q[c];
  // only this wavefront reads its own row of sq; no block barrier needed
  __builtin_amdgcn_wave_barrier();
  const float* Kc = static_cast<const float*>(a.k_cache) + static_cast<size_t>(b) * N * d + h * dh;
  const float* Vc = static_cast<const float*>(a.v_cache) + static_cast<size_t>(b) * N * d + h * dh;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int kb = 0; kb < N; kb += kWave) {
    const int j = kb + lane;
    float s = -INFINITY;
    if (j < N) {
      const float* kr = Kc + static_cast<size_t>(j) * d;
      float acc = 0.f;
      for (int c = 0; c < dh; ++c) acc = fmaf(sq[wid][c], kr[c], acc);
      s = acc * scale2;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(s - m_new);
    l = l * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    const int cnt = min(kWave, N - kb);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = __shfl(p, jj, kWave);
      const float* vr = Vc + static_cast<size_t>(kb + jj) * d;
      if (lane < dh) o0 = fmaf(pj, vr[lane], o0);
      if (lane + kWave < dh) o1 = fmaf(pj, vr[lane + kWave], o1);
    }
    m = m_new;
  }
  float* O = static_cast<float*>(a.o) + (static_cast<size_t>(b) * a.rows_cap + r) * d + h * dh;
  const float inv = 1.0f / l;
  if (lane < dh) O[lane] = o0 * inv;
  if (lane + kWave < dh) O[lane + kWave] = o1 * inv;
}

hipError_t launch_attention(bool bf16, const AttnArgs& a, hipStream_t s, KernelTimer* timer) {
  TimedLaunch t(timer, "attention", s);
  const float scale2 = kLog2e / sqrtf(static_cast<float>(a.dh));
  if (bf16) {
    const dim3 grid((a.rows_cap + kAttnQ - 1) / kAttnQ, a.H, a.B);
    attn_bf16_kernel<<<grid, kAttnThreads, 0, s>>>(a, scale2);
  } else {
    const dim3 grid((a.rows_cap + 3) / 4, a.H, a.B);
    attn_f32_kernel<<<grid, 256, 0, s>>>(a, scale2);
  }
  return hipGetLastError();
}

}  // namespace wamc
