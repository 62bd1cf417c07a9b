// Token scores: action attention mass + latent surprise.
//
// WAM-Cache (paperpeel 2610.11401) §1, §4.2, §4.3 name the two signals:
// the attention the action expert paid to each visual token in the preceding
// chunk, and how far a token's input embedding moved since its last refresh.
// Computed here as
//   P_i = sum_{l,h,a} softmax_j(q_{l,a,h} . K_{l,j,h} / sqrt(dh))[i]
//   U_i = sum_c (z_i,c - zref_i,c)^2
//   score_i = w_a P_i / (L H A) + w_s U_i / sum_j U_j.
//
// P needs the per-query softmax normaliser before any per-key probability
// can be summed, so it is a two-pass computation over the key cache:
//   pass 1 (per (episode, layer*head, key chunk)): each query's running
//           (max, sum of exp) over the chunk's keys -> workspace;
//   pass 2 (same grid): merge the per-chunk (max, sum) of each query,
//           recompute the logits and sum every key's probabilities over the
//           queries -> a [B, L*H, N] partial in workspace;
//   combine 1 (per token block): P_i = fixed-order sum over L*H; U_i by a
//           wavefront reduction over d; per-block partial sums of U;
//   combine 2 (per token block): sum_j U_j from the block partials in fixed
//           order, then the score.
// No float atomics anywhere: results are bitwise reproducible.
//
// bf16 logits run on MFMA (v_mfma_f32_32x32x16_bf16): with A action queries
// the logit work is ~A FLOP per cache byte, far above what VALU fp32 can
// sustain at HBM speed.  Pass 1 uses S^T = K Q^T so each lane owns one query
// and reduces its keys in registers; pass 2 uses S = Q K^T so each lane owns
// one key and reduces its queries in registers.  K fragments are loaded
// straight from HBM into registers (32 bytes of each key row per load
// instruction, the row's two lane halves side by side); the action queries
// of one (layer, head) sit in LDS.
#include "common.h"
#include "launch.h"

namespace wamc {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void merge_ms(float& m, float& z, float m2, float z2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; z = z2; return; }
  const float mn = fmaxf(m, m2);
  z = z * exp2f(m - mn) + z2 * exp2f(m2 - mn);
  m = mn;
}

// ---------------------------------------------------------------------------
// bf16 MFMA passes
// ---------------------------------------------------------------------------

constexpr int kScoreThreads = 256;        // 4 waves
constexpr int kScoreDh = 128;             // head dim of the MFMA path
constexpr int kQaStride = kScoreDh + 8;   // LDS row stride (bf16), breaks bank aliasing
constexpr int kMaxQB = 4;                 // A <= 128

// Fragment slot convention (shared by both MFMA operands, so any fixed
// bijection is valid): lane half h, k-step s, slot j <-> dh = FRAG_DH(h, s) + j.
#ifndef WAMC_SCORE_PAIRED
#define WAMC_SCORE_PAIRED 1
#endif
// 1: dh = s*16 + h*8, so the two lanes of a key read 32 contiguous bytes per
// load instruction (32 cache lines per instruction); 0: dh = h*64 + s*8,
// each lane walking its own 128-byte half row (64 lines per instruction)
__device__ __forceinline__ int frag_dh(int h, int s) { return WAMC_SCORE_PAIRED ? s * 16 + h * 8 : h * 64 + s * 8; }
__device__ __forceinline__ void load_k_frags(const bf16_t* __restrict__ krow, bool valid, int h,
                                             uint4 (&f)[8]) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    f[s] = valid ? *reinterpret_cast<const uint4*>(krow + frag_dh(h, s)) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Stage Qa[l, b, :, h*dh:(h+1)*dh] (A x 128 bf16) into LDS, zero-padding
// rows A..QB*32.  All of a thread's loads are issued before the first LDS
// write, so they are in flight together.
__device__ __forceinline__ void stage_queries(const bf16_t* __restrict__ qa, int A, int QB, int d,
                                              bf16_t* sq) {
  constexpr int kPer = kMaxQB * 32 * (kScoreDh / 8) / kScoreThreads;
  const int chunks = QB * 32 * (kScoreDh / 8);
  uint4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = threadIdx.x + i * kScoreThreads;
    const int row = c / (kScoreDh / 8), col = (c % (kScoreDh / 8)) * 8;
    // rows past A read row 0 (valid memory) and are replaced by zeros
    const uint4 x = *reinterpret_cast<const uint4*>(qa + static_cast<size_t>(row < A ? row : 0) * d + col);
    v[i] = row < A ? x : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = threadIdx.x + i * kScoreThreads;
    const int row = c / (kScoreDh / 8), col = (c % (kScoreDh / 8)) * 8;
    if (c < chunks) *reinterpret_cast<uint4*>(sq + row * kQaStride + col) = v[i];
  }
}

// Each query's softmax (max, sum) over all N keys, from the per-chunk
// partials of pass 1: the QB*32 query slots split the threads into groups
// that take interleaved chunks (8 independent loads per round), then the
// groups' results are merged in group order.  The order is fixed by
// (nchunks, QB), so the result is reproducible.
__device__ __forceinline__ void merge_chunk_stats(const float2* __restrict__ p, int A, int QB, int nchunks,
                                                  float2 (*sg)[kMaxQB * 32], float* smax, float* sinv) {
  const int QS = QB * 32, G = kScoreThreads / QS;
  const int a = threadIdx.x % QS, gi = threadIdx.x / QS;
  float mm = -INFINITY, zz = 0.f;
  if (gi < G && a < A) {
    for (int c0 = gi; c0 < nchunks; c0 += 8 * G) {
      float2 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int cc = c0 + i * G;
        v[i] = cc < nchunks ? p[static_cast<size_t>(cc) * A + a] : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) merge_ms(mm, zz, v[i].x, v[i].y);
    }
  }
  if (gi < G) sg[gi][a] = make_float2(mm, zz);
  __syncthreads();
  if (threadIdx.x < QS) {
    float m = -INFINITY, z = 0.f;
    for (int g = 0; g < G; ++g) merge_ms(m, z, sg[g][threadIdx.x].x, sg[g][threadIdx.x].y);
    const bool real = static_cast<int>(threadIdx.x) < A;
    smax[threadIdx.x] = real ? m : INFINITY;   // padded queries contribute exp2(-inf) = 0
    sinv[threadIdx.x] = real ? 1.f / z : 0.f;
  }
}

__global__ __launch_bounds__(kScoreThreads) void score_pass1_bf16(
    const bf16_t* __restrict__ qa, const bf16_t* __restrict__ kc, int B, int H, int N, int A, int d,
    int chunk_keys, int nchunks, float scale2, float2* __restrict__ ms_out) {
  const int c = blockIdx.x, lh = blockIdx.y, b = blockIdx.z;
  const int l = lh / H, h = lh % H;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, half = lane >> 5, col = lane & 31;
  const int QB = (A + 31) / 32;
  __shared__ bf16_t sq[kMaxQB * 32 * kQaStride];
  __shared__ float2 sms[4][kMaxQB * 32];

  const bf16_t* kbase = kc + (static_cast<size_t>(l) * B + b) * N * d + h * kScoreDh;
  const int k0 = c * chunk_keys, k1 = min(N, k0 + chunk_keys);
  // the first key block's fragments are requested before the queries are
  // staged, so the two memory round trips overlap
  uint4 kf[8];
  {
    const int key = k0 + wid * 32 + col;
    load_k_frags(kbase + static_cast<size_t>(key) * d, key < k1, half, kf);
  }
  stage_queries(qa + (static_cast<size_t>(l) * B + b) * A * d + h * kScoreDh, A, QB, d, sq);
  lds_barrier();

  float m[kMaxQB], z[kMaxQB];
#pragma unroll
  for (int q = 0; q < kMaxQB; ++q) { m[q] = -INFINITY; z[q] = 0.f; }

  for (int kb = k0 + wid * 32; kb < k1; kb += 4 * 32) {
    // prefetch the wave's next key block
    uint4 kn[8];
    const int nkey = kb + 4 * 32 + col;
    load_k_frags(kbase + static_cast<size_t>(nkey) * d, kb + 4 * 32 < k1 && nkey < k1, half, kn);
#pragma unroll
    for (int q = 0; q < kMaxQB; ++q) {
      if (q >= QB) break;
      f32x16_t acc = {};
      const bf16_t* qrow = sq + (q * 32 + col) * kQaStride;
      // the block's query fragments in one batch of LDS reads ahead of the
      // MFMAs (read one by one, each MFMA waited for its own read)
      uint4 qf[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const uint4*>(qrow + frag_dh(half, s));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[s]), as_bf16x8(qf[s]), acc, 0, 0, 0);
      // acc[v]: key kb + (v/4)*8 + half*4 + v%4, query q*32 + col
      float tmax = -INFINITY;
      float sv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = kb + (v / 4) * 8 + half * 4 + (v % 4);
        sv[v] = kk < k1 ? acc[v] * scale2 : -INFINITY;
        tmax = fmaxf(tmax, sv[v]);
      }
      if (tmax != -INFINITY) {
        const float mn = fmaxf(m[q], tmax);
        float zz = m[q] == -INFINITY ? 0.f : z[q] * __builtin_amdgcn_exp2f(m[q] - mn);
#pragma unroll
        for (int v = 0; v < 16; ++v) zz += __builtin_amdgcn_exp2f(sv[v] - mn);
        m[q] = mn;
        z[q] = zz;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = kn[s];
  }
  // merge the two lane halves (same query, different keys), then the waves
#pragma unroll
  for (int q = 0; q < kMaxQB; ++q) {
    const float m2 = __shfl_xor(m[q], 32, kWave), z2 = __shfl_xor(z[q], 32, kWave);
    merge_ms(m[q], z[q], m2, z2);
    if (half == 0 && q < QB) sms[wid][q * 32 + col] = make_float2(m[q], z[q]);
  }
  __syncthreads();
  for (int a = threadIdx.x; a < A; a += kScoreThreads) {
    float mm = -INFINITY, zz = 0.f;
    for (int w = 0; w < 4; ++w) merge_ms(mm, zz, sms[w][a].x, sms[w][a].y);
    ms_out[((static_cast<size_t>(b) * gridDim.y + lh) * nchunks + c) * A + a] = make_float2(mm, zz);
  }
}

__global__ __launch_bounds__(kScoreThreads) void score_pass2_bf16(
    const bf16_t* __restrict__ qa, const bf16_t* __restrict__ kc, int B, int H, int N, int A, int d,
    int chunk_keys, int nchunks, float scale2, const float2* __restrict__ ms_in,
    float* __restrict__ part) {
  const int c = blockIdx.x, lh = blockIdx.y, b = blockIdx.z;
  const int LH = gridDim.y;
  const int l = lh / H, h = lh % H;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, half = lane >> 5, col = lane & 31;
  const int QB = (A + 31) / 32;
  __shared__ bf16_t sq[kMaxQB * 32 * kQaStride];
  __shared__ float smax[kMaxQB * 32], sinv[kMaxQB * 32];
  __shared__ float2 sg[kScoreThreads / 32][kMaxQB * 32];

  const bf16_t* kbase = kc + (static_cast<size_t>(l) * B + b) * N * d + h * kScoreDh;
  float* prow = part + (static_cast<size_t>(b) * LH + lh) * N;
  const int k0 = c * chunk_keys, k1 = min(N, k0 + chunk_keys);
  uint4 kf[8];
  {
    const int key = k0 + wid * 32 + col;
    load_k_frags(kbase + static_cast<size_t>(key) * d, key < k1, half, kf);
  }
  stage_queries(qa + (static_cast<size_t>(l) * B + b) * A * d + h * kScoreDh, A, QB, d, sq);
  merge_chunk_stats(ms_in + (static_cast<size_t>(b) * LH + lh) * nchunks * A, A, QB, nchunks, sg, smax, sinv);
  lds_barrier();

  for (int kb = k0 + wid * 32; kb < k1; kb += 4 * 32) {
    const int key = kb + col;
    uint4 kn[8];
    const int nkey = kb + 4 * 32 + col;
    load_k_frags(kbase + static_cast<size_t>(nkey) * d, kb + 4 * 32 < k1 && nkey < k1, half, kn);
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxQB; ++q) {
      if (q >= QB) break;
      f32x16_t acc = {};
      const bf16_t* qrow = sq + (q * 32 + col) * kQaStride;
      uint4 qf[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const uint4*>(qrow + frag_dh(half, s));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qf[s]), as_bf16x8(kf[s]), acc, 0, 0, 0);
      // acc[v]: query q*32 + (v/4)*8 + half*4 + v%4, key kb + col
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int qq = q * 32 + (v / 4) * 8 + half * 4 + (v % 4);
        sum += __builtin_amdgcn_exp2f(fmaf(acc[v], scale2, -smax[qq])) * sinv[qq];
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = kn[s];
    sum += __shfl_xor(sum, 32, kWave);
    if (half == 0 && key < k1) prow[key] = sum;
  }
}

// ---------------------------------------------------------------------------
// fp32 passes (plain VALU; the small fp32 workloads only)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void score_pass1_f32(
    const float* __restrict__ qa, const float* __restrict__ kc, int B, int H, int N, int A, int d,
    int dh, int chunk_keys, int nchunks, float scale2, float2* __restrict__ ms_out) {
  const int c = blockIdx.x, lh = blockIdx.y, b = blockIdx.z;
  const int l = lh / H, h = lh % H;
  const float* kbase = kc + (static_cast<size_t>(l) * B + b) * N * d + h * dh;
  const int k0 = c * chunk_keys, k1 = min(N, k0 + chunk_keys);
  for (int a = threadIdx.x; a < A; a += blockDim.x) {
    const float* q = qa + ((static_cast<size_t>(l) * B + b) * A + a) * d + h * dh;
    float m = -INFINITY, z = 0.f;
    for (int j = k0; j < k1; ++j) {
      const float* kr = kbase + static_cast<size_t>(j) * d;
      float s = 0.f;
      for (int t = 0; t < dh; ++t) s = fmaf(q[t], kr[t], s);
      merge_ms(m, z, s * scale2, 1.f);
    }
    ms_out[((static_cast<size_t>(b) * gridDim.y + lh) * nchunks + c) * A + a] = make_float2(m, z);
  }
}

__global__ __launch_bounds__(256) void score_pass2_f32(
    const float* __restrict__ qa, const float* __restrict__ kc, int B, int H, int N, int A, int d,
    int dh, int chunk_keys, int nchunks, float scale2, const float2* __restrict__ ms_in,
    float* __restrict__ part) {
  const int c = blockIdx.x, lh = blockIdx.y, b = blockIdx.z;
  const int LH = gridDim.y;
  const int l = lh / H, h = lh % H;
  extern __shared__ float smi[];   // [2 * A]: max, 1/sum
  for (int a = threadIdx.x; a < A; a += blockDim.x) {
    float mm = -INFINITY, zz = 0.f;
    const float2* p = ms_in + (static_cast<size_t>(b) * LH + lh) * nchunks * A + a;
    for (int cc = 0; cc < nchunks; ++cc) merge_ms(mm, zz, p[static_cast<size_t>(cc) * A].x,
                                                  p[static_cast<size_t>(cc) * A].y);
    smi[a] = mm;
    smi[A + a] = 1.f / zz;
  }
  __syncthreads();
  const float* kbase = kc + (static_cast<size_t>(l) * B + b) * N * d + h * dh;
  const int k0 = c * chunk_keys, k1 = min(N, k0 + chunk_keys);
  for (int j = k0 + threadIdx.x; j < k1; j += blockDim.x) {
    const float* kr = kbase + static_cast<size_t>(j) * d;
    float sum = 0.f;
    for (int a = 0; a < A; ++a) {
      const float* q = qa + ((static_cast<size_t>(l) * B + b) * A + a) * d + h * dh;
      float s = 0.f;
      for (int t = 0; t < dh; ++t) s = fmaf(q[t], kr[t], s);
      sum += exp2f(s * scale2 - smi[a]) * smi[A + a];
    }
    part[(static_cast<size_t>(b) * LH + lh) * N + j] = sum;
  }
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------

constexpr int kCombTokens = 16;     // tokens per combine-1 block (4 per wavefront)
constexpr int kCombThreads = 256;

// sum over one 16-byte chunk of (z - zref)^2 (the chunk's bits in a, b; the
// last argument picks the element type)
__device__ __forceinline__ float sq_diff16(uint4 a, uint4 b, bf16_t) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float d0 = __uint_as_float(wa[i] << 16) - __uint_as_float(wb[i] << 16);
    const float d1 = __uint_as_float(wa[i] & 0xffff0000u) - __uint_as_float(wb[i] & 0xffff0000u);
    acc = fmaf(d0, d0, acc);
    acc = fmaf(d1, d1, acc);
  }
  return acc;
}
__device__ __forceinline__ float sq_diff16(uint4 ua, uint4 ub, float) {
  const float4 a = __builtin_bit_cast(float4, ua);
  const float4 b = __builtin_bit_cast(float4, ub);
  const float d0 = a.x - b.x, d1 = a.y - b.y, d2 = a.z - b.z, d3 = a.w - b.w;
  return fmaf(d0, d0, fmaf(d1, d1, fmaf(d2, d2, d3 * d3)));
}

template <typename T>
__global__ __launch_bounds__(kCombThreads) void score_combine1(
    const float* __restrict__ part, int LH, const float* __restrict__ mass_in,
    const T* __restrict__ z, const T* __restrict__ zref, int N, int d,
    float* __restrict__ mass, float* __restrict__ surprise, float* __restrict__ usum_blocks) {
  constexpr int kPer = 16 / sizeof(T);   // elements per 16-byte chunk
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kCombTokens;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ float sp[16][kCombTokens];
  __shared__ float su[kCombTokens];

  // P: 16 interleaved groups of the L*H partial rows, combined in fixed order
  {
    const int tk = tid & (kCombTokens - 1), grp = tid / kCombTokens;
    const int tok = t0 + tk;
    float acc = 0.f;
    if (tok < N) {
      if (mass_in) {
        if (grp == 0) acc = mass_in[static_cast<size_t>(b) * N + tok];
      } else {
        // rows grp, grp+16, ... summed in that order; 8 loads in flight at a time
        for (int r0 = grp; r0 < LH; r0 += 16 * 8) {
          float v[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int r = r0 + 16 * q;
            v[q] = r < LH ? part[(static_cast<size_t>(b) * LH + r) * N + tok] : 0.f;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) acc += v[q];
        }
      }
    }
    sp[grp][tk] = acc;
  }
  // U: each wavefront takes 4 tokens, lanes stride over 16-byte chunks
  const int chunks = d / kPer;
  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = t0 + wid * 4 + j;
    float acc = 0.f;
    if (tok < N) {
      const T* zr = z + (static_cast<size_t>(b) * N + tok) * d;
      const T* rr = zref + (static_cast<size_t>(b) * N + tok) * d;
      // chunks lane, lane+64, ... in that order; 4 pairs of loads in flight at a time
      for (int c0 = lane; c0 < chunks; c0 += 4 * kWave) {
        uint4 za[4], ra[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = c0 + q * kWave < chunks ? c0 + q * kWave : c0;
          za[q] = *reinterpret_cast<const uint4*>(zr + c * kPer);
          ra[q] = *reinterpret_cast<const uint4*>(rr + c * kPer);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c0 + q * kWave < chunks) acc += sq_diff16(za[q], ra[q], T{});
      }
    }
    u[j] = acc;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float v = wave_sum(u[j]);
    if (lane == 0) su[wid * 4 + j] = v;
  }
  __syncthreads();
  if (tid < kCombTokens) {
    const int tok = t0 + tid;
    float p = 0.f;
#pragma unroll
    for (int gi = 0; gi < 16; ++gi) p += sp[gi][tid];
    if (tok < N) {
      mass[static_cast<size_t>(b) * N + tok] = p;
      surprise[static_cast<size_t>(b) * N + tok] = su[tid];
    }
  }
  if (wid == 0) {
    const float v = lane < kCombTokens && t0 + lane < N ? su[lane] : 0.f;
    const float bs = wave_sum(v);
    if (lane == 0) usum_blocks[static_cast<size_t>(b) * gridDim.x + blockIdx.x] = bs;
  }
}

__global__ __launch_bounds__(256) void score_combine2(
    const float* __restrict__ mass, const float* __restrict__ surprise,
    const float* __restrict__ usum_blocks, int nblocks, int N, float w_attn_norm, float w_surprise,
    float* __restrict__ score, float* __restrict__ mass_out, float* __restrict__ surprise_out) {
  const int b = blockIdx.y;
  __shared__ float red[4];
  const float total = usum_total(usum_blocks + static_cast<size_t>(b) * nblocks, nblocks, red);
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const size_t o = static_cast<size_t>(b) * N + i;
  const float p = mass[o], u = surprise[o];
  score[o] = combine_score(p, u, total, w_attn_norm, w_surprise);
  if (mass_out) mass_out[o] = p;
  if (surprise_out) surprise_out[o] = u;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

ScorePlan plan_score(int B, int L, int H, int N, int A, bool bf16) {
  ScorePlan p;
  const long long keys = static_cast<long long>(N) * L * H * B;
  int ck;
  if (bf16) {
    // aim for ~2048 workgroups; chunks are whole 128-key wave rounds
    long long want = (keys + 2047) / 2048;
    ck = static_cast<int>(((want + 127) / 128) * 128);
    if (ck < 128) ck = 128;
    if (ck > 2048) ck = 2048;
  } else {
    ck = 256;
  }
  p.chunk_keys = ck;
  p.nchunks = (N + ck - 1) / ck;
  p.comb_blocks = (N + kCombTokens - 1) / kCombTokens;
  p.ms_bytes = static_cast<size_t>(B) * L * H * p.nchunks * A * sizeof(float2);
  p.part_bytes = static_cast<size_t>(B) * L * H * N * sizeof(float);
  p.tok_bytes = static_cast<size_t>(B) * N * sizeof(float);
  p.usum_bytes = static_cast<size_t>(B) * p.comb_blocks * sizeof(float);
  return p;
}

hipError_t launch_score_mass(bool bf16, const void* qa, const void* kc, int B, int L, int H, int N,
                             int A, int d, const ScorePlan& p, float2* ms, float* part,
                             hipStream_t s, KernelTimer* timer) {
  const int dh = d / H;
  const float scale2 = kLog2e / sqrtf(static_cast<float>(dh));
  const dim3 grid(p.nchunks, L * H, B);
  if (bf16) {
    {
      TimedLaunch t(timer, "score_pass1", s);
      launch(score_pass1_bf16, grid, kScoreThreads, 0, s, static_cast<const bf16_t*>(qa),
          static_cast<const bf16_t*>(kc), B, H, N, A, d, p.chunk_keys, p.nchunks, scale2, ms);
    }
    TimedLaunch t(timer, "score_pass2", s);
    launch(score_pass2_bf16, grid, kScoreThreads, 0, s, static_cast<const bf16_t*>(qa),
        static_cast<const bf16_t*>(kc), B, H, N, A, d, p.chunk_keys, p.nchunks, scale2, ms, part);
  } else {
    {
      TimedLaunch t(timer, "score_pass1", s);
      launch(score_pass1_f32, grid, 256, 0, s, static_cast<const float*>(qa), static_cast<const float*>(kc),
          B, H, N, A, d, dh, p.chunk_keys, p.nchunks, scale2, ms);
    }
    TimedLaunch t(timer, "score_pass2", s);
    launch(score_pass2_f32, grid, 256, 2 * A * sizeof(float), s, static_cast<const float*>(qa),
        static_cast<const float*>(kc), B, H, N, A, d, dh, p.chunk_keys, p.nchunks, scale2, ms, part);
  }
  return hipGetLastError();
}

hipError_t launch_score_partials(bool bf16, const float* part, int LH, const float* mass_in, const void* z,
                                 const void* zref, int B, int N, int d, const ScorePlan& p, float* mass_tmp,
                                 float* surprise_tmp, float* usum, hipStream_t s, KernelTimer* timer) {
  TimedLaunch t(timer, "score_combine", s);
  const dim3 grid(p.comb_blocks, B);
  if (bf16)
    launch(score_combine1<bf16_t>, grid, kCombThreads, 0, s, part, LH, mass_in, static_cast<const bf16_t*>(z),
        static_cast<const bf16_t*>(zref), N, d, mass_tmp, surprise_tmp, usum);
  else
    launch(score_combine1<float>, grid, kCombThreads, 0, s, part, LH, mass_in, static_cast<const float*>(z),
        static_cast<const float*>(zref), N, d, mass_tmp, surprise_tmp, usum);
  return hipGetLastError();
}

hipError_t launch_score_finish(const float* mass_tmp, const float* surprise_tmp, const float* usum, int B, int N,
                               float w_attn_norm, float w_surprise, const ScorePlan& p, float* score,
                               float* mass_out, float* surprise_out, hipStream_t s, KernelTimer* timer) {
  TimedLaunch t(timer, "score_combine", s);
  launch(score_combine2, dim3((N + 255) / 256, B), 256, 0, s, mass_tmp, surprise_tmp, usum, p.comb_blocks, N,
      w_attn_norm, w_surprise, score, mass_out, surprise_out);
  return hipGetLastError();
}

}  // namespace wamc
