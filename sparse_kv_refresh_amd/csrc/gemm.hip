// Projections of the refreshed rows: C = A W^T with fused epilogues.
//
// WAM-Cache (paperpeel 2610.11401) §3: Q, K and V are linear projections of
// the module input and the module applies an MLP, each sub-layer with a
// residual.  Only the k_eff refreshed rows go through these GEMMs, which is
// where the refresh saves its FLOPs (§5.2: prefill cost scales with the
// recompute ratio).
//
// Epilogues (applied to acc + bias, all in f32):
//   EPI_QKV   : Q -> q_out (act), K/V -> written straight into this layer's
//               cache at the row's token index (the scatter is fused here);
//   EPI_RESID_OUT / EPI_RESID_DOWN : out = in + gate * v   (gated residual, f32 stream);
//   EPI_GELU  : g = act(GELU_erf(v));
//   EPI_KV    : text keys/values of the cross-attention (K -> k_cache, V -> v_cache rows);
//   EPI_STORE : g = act(v)  (the cross-attention queries);
//   EPI_RESID_PLAIN : out = in + v  (the ungated cross-attention residual).
//
// bf16 path (K % 64 == 0): BM x BN tiles (128x128, 128x256 or 256x128,
// picked per GEMM shape), 4 waves in a 2x2 layout, each wave (BM/2) x (BN/2)
// as blocks of v_mfma_f32_32x32x16_bf16.  Global tiles go straight into LDS
// (global_load_lds_dwordx4), STAGES k-tiles in flight, one s_barrier per
// k-tile.  The tile order is XCD-aware: consecutive workgroup ids go
// round-robin over the 8 XCDs, so ids are remapped to give each XCD a
// contiguous range of tiles, then grouped 8 row-tiles at a time so tiles that
// share weight columns run close together in the same L2.  A register-staged
// 128x128 kernel with padded LDS rows covers K % 64 != 0.
// fp32 path: 64x64x16 LDS tiles on VALU FMAs (correctness path for the small
// fp32 workloads).
#include "common.h"
#include "launch.h"
#include "rowops.h"

#include <algorithm>

namespace wamc {

// ---------------------------------------------------------------------------
// shared epilogue
// ---------------------------------------------------------------------------

// Runs CALL with the compile-time epilogue E of the run-time kind epi.
#define WAMC_EPI_DISPATCH(epi, CALL)                                      \
  switch (epi) {                                                          \
    case EPI_QKV: { constexpr int E = EPI_QKV; CALL; } break;             \
    case EPI_RESID_OUT: { constexpr int E = EPI_RESID_OUT; CALL; } break; \
    case EPI_GELU: { constexpr int E = EPI_GELU; CALL; } break;           \
    case EPI_RESID_DOWN: { constexpr int E = EPI_RESID_DOWN; CALL; } break; \
    case EPI_KV: { constexpr int E = EPI_KV; CALL; } break;               \
    case EPI_STORE: { constexpr int E = EPI_STORE; CALL; } break;         \
    case EPI_RESID_PLAIN: { constexpr int E = EPI_RESID_PLAIN; CALL; } break; \
  }

struct RowInfo {
  bool valid;
  int b, r;
};

__device__ __forceinline__ RowInfo row_info(const GemmArgs& g, int m) {
  RowInfo ri;
  ri.b = m / g.rows_cap;
  ri.r = m - ri.b * g.rows_cap;
  ri.valid = m < g.M && ri.r < rows_of(g.k_eff, ri.b, g.rows_cap);
  return ri;
}

template <int EPI, typename T>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const RowInfo& ri, int m, int n, float acc) {
  if (!ri.valid || n >= g.Nout) return;
  const float v = acc + Elem<T>::load(static_cast<const T*>(g.bias), n);
  if constexpr (EPI == EPI_QKV || EPI == EPI_KV) {
    const int d = g.d_model;
    const int wr = n / d, c = n - wr * d;
    const int which = wr + (EPI == EPI_KV ? 1 : 0);
    if (which == 0) {
      Elem<T>::store(static_cast<T*>(g.q_out), static_cast<size_t>(m) * d + c, v);
    } else {
      const int tok = g.idx ? g.idx[static_cast<size_t>(ri.b) * g.n_tokens + ri.r] : ri.r;
      if (tok < 0 || tok >= g.n_tokens) return;
      T* cache = static_cast<T*>(which == 1 ? g.k_cache : g.v_cache);
      Elem<T>::store(cache, (static_cast<size_t>(ri.b) * g.n_tokens + tok) * d + c, v);
    }
  } else if constexpr (EPI == EPI_RESID_OUT || EPI == EPI_RESID_DOWN) {
    const size_t o = static_cast<size_t>(m) * g.Nout + n;
    g.resid_out[o] = g.resid_in[o] + Elem<T>::load(static_cast<const T*>(g.gate), n) * v;
  } else if constexpr (EPI == EPI_RESID_PLAIN) {
    const size_t o = static_cast<size_t>(m) * g.Nout + n;
    g.resid_out[o] = g.resid_in[o] + v;
  } else if constexpr (EPI == EPI_STORE) {
    Elem<T>::store(static_cast<T*>(g.g_out), static_cast<size_t>(m) * g.Nout + n, v);
  } else {
    Elem<T>::store(static_cast<T*>(g.g_out), static_cast<size_t>(m) * g.Nout + n, gelu_erf(v));
  }
}

// The Q / K / V output a chunk of columns goes to.  The three pointers pass
// through an empty asm statement first: a per-thread select between fields of
// the kernel argument block is otherwise compiled into a per-thread load of
// the selected field, and every store then waits for that load and, since
// stores share its counter, for all the stores before it.
typedef __attribute__((address_space(1))) bf16_t gbf16_t;   // in global memory
typedef unsigned u32x4_v __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x4_v gu32x4_t;
typedef __attribute__((address_space(1))) u32x2_v gu32x2_t;
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) f32x4_v gf32x4_t;
struct QkvDst {
  gbf16_t *q, *k, *v;
};
__device__ __forceinline__ QkvDst qkv_dst(const GemmArgs& g) {
  // typed as global pointers, so the stores stay global (not flat) stores
  gbf16_t* q = (gbf16_t*)g.q_out;
  gbf16_t* k = (gbf16_t*)g.k_cache;
  gbf16_t* v = (gbf16_t*)g.v_cache;
  asm("" : "+s"(q), "+s"(k), "+s"(v));
  return {q, k, v};
}
__device__ __forceinline__ gbf16_t* qkv_pick(const QkvDst& p, int which) {
  return which == 0 ? p.q : (which == 1 ? p.k : p.v);
}

// true when no row of [m0, m0 + rows) is valid (the whole tile can exit)
__device__ __forceinline__ bool tile_empty(const GemmArgs& g, int m0, int rows) {
  if (m0 >= g.M) return true;
  if (!g.k_eff) return false;
  const int m1 = min(g.M, m0 + rows) - 1;
  const int b0 = m0 / g.rows_cap, b1 = m1 / g.rows_cap;
  for (int b = b0; b <= b1; ++b) {
    const int lo = b == b0 ? m0 - b * g.rows_cap : 0;
    if (lo < rows_of(g.k_eff, b, g.rows_cap)) return false;
  }
  return true;
}

// XCD-aware remap of a linear workgroup id, then grouped (GM row-tiles)
// ordering over a tiles_m x tiles_n grid.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int id = xcd_remap(pid, tiles_m * tiles_n);
  const int group = id / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = id - group * GM * tiles_n;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsK = kBK + 8;   // padded LDS row (bf16 elements)
constexpr int kGemmThreads = 256;
#ifndef WAMC_GEMM_STAGES
#define WAMC_GEMM_STAGES 2
#endif
#ifndef WAMC_GEMM_BK
#define WAMC_GEMM_BK 64
#endif
constexpr int kGemmStages = WAMC_GEMM_STAGES;
constexpr int kDtlBK = WAMC_GEMM_BK;
#ifndef WAMC_GEMM_GENERIC
#define WAMC_GEMM_GENERIC 0
#endif
constexpr bool kForceGeneric = WAMC_GEMM_GENERIC != 0;

// ---------------------------------------------------------------------------
// tile epilogue of the bf16 kernels
//
// One pass over the 128 rows of the tile fills a row table in LDS (row
// validity, the episode/row split and, for QKV, the cache row of the row's
// token), so the per-element work is a table read, the bias and the store.
// ---------------------------------------------------------------------------

template <int EPI, int BM, int NT = kGemmThreads>
__device__ __forceinline__ void fill_row_table(const GemmArgs& g, int m0, int* tab, int mend = 0x7fffffff) {
  for (int t = threadIdx.x; t < BM; t += NT) {
    const int m = m0 + t;
    const RowInfo ri = row_info(g, m);
    int r0 = -1, r1 = -1;
    if (ri.valid && m < mend) {
      r0 = m;
      if constexpr (EPI == EPI_QKV || EPI == EPI_KV) {
        const int tok = g.idx ? g.idx[static_cast<size_t>(ri.b) * g.n_tokens + ri.r] : ri.r;
        r1 = (tok >= 0 && tok < g.n_tokens) ? ri.b * g.n_tokens + tok : -1;
      }
    }
    tab[t] = r0;
    tab[BM + t] = r1;
  }
}

// The bf16 kernels issue the MFMA with the weight fragment as operand A and
// the activation fragment as operand B, i.e. they compute C^T blocks.  In the
// 32x32 output layout that gives lane (half, col) ONE output row per block
//   lr = wm*WTM + i*32 + col
// and, for element group g (v = 4g..4g+3), FOUR consecutive output columns
//   n = n0 + wn*WTN + j*32 + g*8 + half*4 + (0..3).
// Stored from that layout, one store instruction would touch 32 rows with 8
// or 16 bytes each.  So the epilogue goes through LDS, one 32-row block per
// wave row at a time: the waves holding accumulators write them (raw f32)
// into a [WGM*32][BN+4] staging tile, then all NT threads of the workgroup
// take 16-byte row chunks of it, apply bias / GELU / gate and residual with
// loads of whole rows, and store whole rows.  The arithmetic per element is
// the same as element-wise: v = acc + bias; out = act(v), or
// out = resid + gate * v (one fma).
template <int BM, int BN, int WTM>
constexpr int epi_stage_bytes() {
  return (BM / WTM) * 32 * (BN + 4) * 4;
}

template <int EPI, int BM, int BN, int TI, int TJ, int WTM, int WTN, int NT>
__device__ __forceinline__ void tile_epilogue_staged(const GemmArgs& g, const f32x16_t (&acc)[TI][TJ], int n0, int wm,
                                              int wn, int half, int col, const int* tab, float* stage, bool writer) {
  constexpr int WGM = BM / WTM;
  constexpr int SROWS = WGM * 32;          // staged rows per step
  constexpr int SSTRIDE = BN + 4;          // floats; breaks bank aliasing of the row-wise writes
  constexpr bool F32OUT = EPI == EPI_RESID_OUT || EPI == EPI_RESID_DOWN || EPI == EPI_RESID_PLAIN;
  constexpr int EPC = F32OUT ? 4 : 8;      // output elements per 16-byte chunk
  constexpr int CPR = BN / EPC;            // chunks per row
  constexpr int PER = SROWS * CPR / NT;    // chunks per thread per step
  static_assert(PER * NT == SROWS * CPR && PER >= 1, "epilogue chunks / threads");
  // When NT % CPR == 0 a thread's chunks q = tid + p*NT all sit in column
  // chunk tid % CPR, and its bias and gate are loaded once for the tile;
  // otherwise per chunk, as it is stored.
  constexpr bool FIXC = NT % CPR == 0;
  const int tid = threadIdx.x;
  const int d = g.d_model;
  const bf16_t* bias = static_cast<const bf16_t*>(g.bias);
  const QkvDst qd = qkv_dst(g);
  auto chunk_cols = [&](int q, int& nc, bool& nok, float (&bsv)[EPC], float (&gt)[4]) {
    const int n = n0 + (q % CPR) * EPC;
    nok = n < g.Nout;   // Nout % 8 == 0: a chunk lies wholly inside or outside
    nc = nok ? n : 0;
    if constexpr (EPC == 8) {
      const uint4 bb = *reinterpret_cast<const uint4*>(bias + nc);
      const uint32_t w[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bsv[2 * e] = __uint_as_float(w[e] << 16);
        bsv[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
      const uint2 bb = *reinterpret_cast<const uint2*>(bias + nc);
      bsv[0] = __uint_as_float(bb.x << 16); bsv[1] = __uint_as_float(bb.x & 0xffff0000u);
      bsv[2] = __uint_as_float(bb.y << 16); bsv[3] = __uint_as_float(bb.y & 0xffff0000u);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) gt[e] = 1.f;   // EPI_RESID_PLAIN: ungated
    if constexpr (EPI == EPI_RESID_OUT || EPI == EPI_RESID_DOWN) {
      const uint2 gg = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(g.gate) + nc);
      gt[0] = __uint_as_float(gg.x << 16); gt[1] = __uint_as_float(gg.x & 0xffff0000u);
      gt[2] = __uint_as_float(gg.y << 16); gt[3] = __uint_as_float(gg.y & 0xffff0000u);
    }
  };
  int nc0 = 0;
  bool nok0 = false;
  float bsv0[EPC], gt0[4];
  if constexpr (FIXC) chunk_cols(tid, nc0, nok0, bsv0, gt0);
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    // phase 1: raw accumulators of rows wm*WTM + i*32 + col -> staging row wm*32 + col
    if (writer) {
      float* srow = stage + (wm * 32 + col) * SSTRIDE + wn * WTN + half * 4;
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
          *reinterpret_cast<float4*>(srow + j * 32 + gg * 8) =
              make_float4(acc[i][j][4 * gg + 0], acc[i][j][4 * gg + 1], acc[i][j][4 * gg + 2], acc[i][j][4 * gg + 3]);
    }
    __syncthreads();
    // phase 2: chunk q = tid + p*NT -> staging row sr = q / CPR.  Every load
    // of the step (staged values, row table, residual rows) is issued before
    // the first store: a store to an output that may alias them would
    // otherwise hold each chunk's loads behind the previous chunk's store.
    float v[PER][EPC];
    int rr[PER], rq[PER];
    float4 xin[F32OUT ? PER : 1];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int sr = (tid + p * NT) / CPR;
      rr[p] = (sr / 32) * WTM + i * 32 + (sr % 32);   // row within the tile
      rq[p] = tab[rr[p]];
      const float* sp = stage + sr * SSTRIDE + ((tid + p * NT) % CPR) * EPC;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(sp + e);
        v[p][e] = x.x; v[p][e + 1] = x.y; v[p][e + 2] = x.z; v[p][e + 3] = x.w;
      }
    }
    if constexpr (F32OUT) {
#pragma unroll
      for (int p = 0; p < PER; ++p)
        xin[p] = *reinterpret_cast<const float4*>(g.resid_in + static_cast<size_t>(rq[p] < 0 ? 0 : rq[p]) * g.Nout +
                                                  (FIXC ? nc0 : min(n0 + ((tid + p * NT) % CPR) * EPC, g.Nout - EPC)));
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int nc = nc0;
      bool nok = nok0;
      float bsv[EPC], gt[4];
      if constexpr (FIXC) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) bsv[e] = bsv0[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) gt[e] = gt0[e];
      } else {
        chunk_cols(tid + p * NT, nc, nok, bsv, gt);
      }
      if constexpr (F32OUT) {
        float4 xo;
        xo.x = fmaf(gt[0], v[p][0] + bsv[0], xin[p].x);
        xo.y = fmaf(gt[1], v[p][1] + bsv[1], xin[p].y);
        xo.z = fmaf(gt[2], v[p][2] + bsv[2], xin[p].z);
        xo.w = fmaf(gt[3], v[p][3] + bsv[3], xin[p].w);
        if (rq[p] >= 0 && nok)
          *reinterpret_cast<float4*>(g.resid_out + static_cast<size_t>(rq[p]) * g.Nout + nc) = xo;
      } else {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[e] = v[p][e] + bsv[e];
          if constexpr (EPI == EPI_GELU) y[e] = gelu_erf_fast(y[e]);
        }
        uint4 w;
        w.x = pack_bf16x2(y[0], y[1]);
        w.y = pack_bf16x2(y[2], y[3]);
        w.z = pack_bf16x2(y[4], y[5]);
        w.w = pack_bf16x2(y[6], y[7]);
        if constexpr (EPI == EPI_QKV || EPI == EPI_KV) {
          // a chunk of 8 columns lies in one of Q | K | V (d % 8 == 0)
          const int wr = nc / d, c = nc - wr * d;
          const int which = wr + (EPI == EPI_KV ? 1 : 0);
          const int r = which == 0 ? rq[p] : tab[BM + rr[p]];
          gbf16_t* dst = qkv_pick(qd, which);
          if (r >= 0 && nok) *reinterpret_cast<gu32x4_t*>(dst + static_cast<size_t>(r) * d + c) = __builtin_bit_cast(u32x4_v, w);
        } else {
          if (rq[p] >= 0 && nok)
            *reinterpret_cast<uint4*>(static_cast<bf16_t*>(g.g_out) + static_cast<size_t>(rq[p]) * g.Nout + nc) = w;
        }
      }
    }
    __syncthreads();   // the next step's staging overwrites these rows
  }
}

// Element-wise store from the MFMA layout (see above): one row per lane and
// block, four consecutive columns per element group.
template <int EPI, int BM, int BN, int TI, int TJ, int WTM, int WTN>
__device__ __forceinline__ void tile_epilogue_direct(const GemmArgs& g, const f32x16_t (&acc)[TI][TJ], int m0, int n0,
                                              int wm, int wn, int half, int col, const int* tab) {
  (void)m0;
  // The lane's TJ*4 column groups.  Nout % 4 == 0, so a group lies wholly
  // inside or outside [0, Nout); groups outside read column 0 (valid memory)
  // and store nothing.  Every load is unconditional, so all of a row block's
  // loads are in flight together instead of one round trip per group.
  constexpr int NG = TJ * 4;
  const bf16_t* bias = static_cast<const bf16_t*>(g.bias);
  const QkvDst qd = qkv_dst(g);
  int ncol[NG];
  bool nok[NG];
  uint2 bb[NG];
#pragma unroll
  for (int jg = 0; jg < NG; ++jg) {
    const int n = n0 + wn * WTN + (jg / 4) * 32 + (jg % 4) * 8 + half * 4;
    nok[jg] = n < g.Nout;
    ncol[jg] = nok[jg] ? n : 0;
    bb[jg] = *reinterpret_cast<const uint2*>(bias + ncol[jg]);
  }
  // gate of the gated residuals (EPI_RESID_PLAIN: 1.0 = 0x3f80 in bf16)
  uint2 gt[NG];
#pragma unroll
  for (int jg = 0; jg < NG; ++jg) {
    if constexpr (EPI == EPI_RESID_OUT || EPI == EPI_RESID_DOWN)
      gt[jg] = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(g.gate) + ncol[jg]);
    else
      gt[jg] = make_uint2(0x3f803f80u, 0x3f803f80u);
  }
  auto biased = [&](int i, int jg, int e) {
    const uint32_t w = e < 2 ? bb[jg].x : bb[jg].y;
    const float b = (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    return acc[i][jg / 4][4 * (jg % 4) + e] + b;
  };
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    // one row block at a time: hoisting the residual loads of every block
    // at once costs more registers than the large tiles have
    __builtin_amdgcn_sched_barrier(0);
    const int lr = wm * WTM + i * 32 + col;
    const int rq = tab[lr];
    if constexpr (EPI == EPI_QKV || EPI == EPI_KV) {
      const int rkv = tab[BM + lr];
      const int d = g.d_model;
      // a tile crosses at most one of the Q|K|V boundaries (BN <= 256 <= 2d)
      const int which0 = n0 / d, edge = (which0 + 1) * d;
      constexpr int kOff = EPI == EPI_KV ? 1 : 0;   // EPI_KV has no Q columns
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) {
        const int n = ncol[jg];
        const int wr = which0 + (n >= edge ? 1 : 0), c = n - wr * d;
        const int which = wr + kOff;
        const int r = which == 0 ? rq : rkv;
        uint2 w;
        w.x = pack_bf16x2(biased(i, jg, 0), biased(i, jg, 1));
        w.y = pack_bf16x2(biased(i, jg, 2), biased(i, jg, 3));
        gbf16_t* dst = qkv_pick(qd, which);
        if (r >= 0 && nok[jg]) *reinterpret_cast<gu32x2_t*>(dst + static_cast<size_t>(r) * d + c) = __builtin_bit_cast(u32x2_v, w);
      }
    } else if constexpr (EPI == EPI_RESID_OUT || EPI == EPI_RESID_DOWN || EPI == EPI_RESID_PLAIN) {
      const size_t rbase = static_cast<size_t>(rq < 0 ? 0 : rq) * g.Nout;
      float4 xin[NG];
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) xin[jg] = *reinterpret_cast<const float4*>(g.resid_in + rbase + ncol[jg]);
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) {
        float4 xo;
        xo.x = fmaf(__uint_as_float(gt[jg].x << 16), biased(i, jg, 0), xin[jg].x);
        xo.y = fmaf(__uint_as_float(gt[jg].x & 0xffff0000u), biased(i, jg, 1), xin[jg].y);
        xo.z = fmaf(__uint_as_float(gt[jg].y << 16), biased(i, jg, 2), xin[jg].z);
        xo.w = fmaf(__uint_as_float(gt[jg].y & 0xffff0000u), biased(i, jg, 3), xin[jg].w);
        if (rq >= 0 && nok[jg]) *reinterpret_cast<float4*>(g.resid_out + rbase + ncol[jg]) = xo;
      }
    } else {
      bf16_t* out = static_cast<bf16_t*>(g.g_out) + static_cast<size_t>(rq < 0 ? 0 : rq) * g.Nout;
#pragma unroll
      for (int jg = 0; jg < NG; ++jg) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = biased(i, jg, e);
          if constexpr (EPI == EPI_GELU) v[e] = gelu_erf_fast(v[e]);
        }
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        if (rq >= 0 && nok[jg]) *reinterpret_cast<uint2*>(out + ncol[jg]) = w;
      }
    }
  }
}

// Epilogue choice (measured at d = 1536): staging pays for the QKV epilogue,
// whose K/V rows scatter to cache rows (QKV 55 -> 51 us at 2458 rows); for
// the residual epilogues it breaks even and for GELU it costs 4 us, so those
// store from the MFMA layout directly.
template <int EPI, int BM, int BN, int TI, int TJ, int WTM, int WTN, int NT>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& g, const f32x16_t (&acc)[TI][TJ], int m0, int n0,
                                              int wm, int wn, int half, int col, const int* tab, float* stage,
                                              bool writer) {
  if constexpr (EPI == EPI_QKV || EPI == EPI_KV) {
    tile_epilogue_staged<EPI, BM, BN, TI, TJ, WTM, WTN, NT>(g, acc, n0, wm, wn, half, col, tab, stage, writer);
  } else {
    if (writer) tile_epilogue_direct<EPI, BM, BN, TI, TJ, WTM, WTN>(g, acc, m0, n0, wm, wn, half, col, tab);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x8_t frag(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_bf16_kernel(GemmArgs g) {
  const int tiles_m = (g.M + kBM - 1) / kBM, tiles_n = (g.Nout + kBN - 1) / kBN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  if (tile_empty(g, m0, kBM)) return;

  __shared__ __attribute__((aligned(16))) bf16_t As[2][kBM * kLdsK];
  __shared__ __attribute__((aligned(16))) bf16_t Ws[2][kBN * kLdsK];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int half = lane >> 5, col = lane & 31;
  const bf16_t* A = static_cast<const bf16_t*>(g.a);
  const bf16_t* W = static_cast<const bf16_t*>(g.w);
  const int K = g.K;

  // each thread moves 4 16-byte chunks of A and 4 of W per k-tile
  uint4 ra[4], rw[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = tid + i * kGemmThreads;
      const int row = chunk >> 3, kc = (chunk & 7) * 8;
      const int gk = k0 + kc;
      const int am = m0 + row, wn_ = n0 + row;
      ra[i] = (am < g.M && gk < K) ? *reinterpret_cast<const uint4*>(A + static_cast<size_t>(am) * K + gk)
                                   : make_uint4(0, 0, 0, 0);
      rw[i] = (wn_ < g.Nout && gk < K) ? *reinterpret_cast<const uint4*>(W + static_cast<size_t>(wn_) * K + gk)
                                      : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = tid + i * kGemmThreads;
      const int row = chunk >> 3, kc = (chunk & 7) * 8;
      *reinterpret_cast<uint4*>(&As[buf][row * kLdsK + kc]) = ra[i];
      *reinterpret_cast<uint4*>(&Ws[buf][row * kLdsK + kc]) = rw[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  const int nk = (K + kBK - 1) / kBK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * kBK);
    const bf16_t* as = &As[cur][(wm * 64 + col) * kLdsK + half * 8];
    const bf16_t* ws = &Ws[cur][(wn * 64 + col) * kLdsK + half * 8];
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const bf16x8_t a0 = frag(as + s * 16), a1 = frag(as + 32 * kLdsK + s * 16);
      const bf16x8_t b0 = frag(ws + s * 16), b1 = frag(ws + 32 * kLdsK + s * 16);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, a0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, a0, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, a1, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, a1, acc[1][1], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

  int* tab = reinterpret_cast<int*>(&As[0][0]);   // the last k-tile ended with a barrier
  fill_row_table<EPI, kBM>(g, m0, tab);
  __syncthreads();
  static_assert(epi_stage_bytes<kBM, kBN, kBM / 2>() <= sizeof(Ws), "epilogue staging fits the W tiles");
  tile_epilogue<EPI, kBM, kBN, 2, 2, kBM / 2, kBN / 2, kGemmThreads>(g, acc, m0, n0, wm, wn, half, col, tab,
                                                                     reinterpret_cast<float*>(&Ws[0][0]), true);
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM with direct-to-LDS loads (K % 64 == 0)
//
// Global tiles go straight into LDS with global_load_lds_dwordx4 (no VGPR
// staging), STAGES k-tiles in flight in a ring of LDS buffers.  A direct-to-
// LDS instruction writes 16 bytes per lane at consecutive LDS addresses, so
// the tile layout in LDS is chosen by *which* global chunk each lane fetches:
// chunk (row, kc) of a tile lives at LDS chunk row*CPR + swz_kc(row, kc), an
// XOR swizzle under which the rows of an MFMA fragment read hit distinct
// banks.  Rows past M / Nout load a clamped (valid) row whose
// results are never stored.
// ---------------------------------------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N) with expcnt / lgkmcnt left at their maxima (gfx9 encoding)
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(ahead * LOADS) for a run-time ahead in [0, MAXA]
template <int LOADS, int MAXA>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  if constexpr (MAXA <= 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= MAXA) wait_vmcnt<MAXA * LOADS>();
    else wait_tiles_ahead<LOADS, MAXA - 1>(ahead);
  }
}

// Column key of element chunk (row, kc) in a tile with CPR 16-byte chunks per
// row.  gfx950 LDS has 64 banks (a 256-byte window) and serves ds_read_b128
// 16 lanes at a time; an MFMA fragment read has 16 consecutive rows at the
// same kc in each phase, so the XOR key makes those 16 rows land in 16
// different 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int swz_kc(int row, int kc) {
  if constexpr (CPR == 8) return kc ^ ((row >> 1) & 7);   // 128-byte rows: 2 rows per window
  else return kc ^ ((row >> 2) & 3);                      // 64-byte rows: 4 rows per window
}
template <int CPR>
__device__ __forceinline__ int swz(int row, int kc) {
  return row * CPR + swz_kc<CPR>(row, kc);
}

// One BK-deep stage of a wave's TI x TJ block of 32x32 tiles, A rows from
// `as`, W rows from `ws`.  The fragments of k-step s+1 are read before the
// MFMAs of step s issue (the scheduling fence keeps that order), so their LDS
// latency runs under those MFMAs.
template <int BK, int TI, int TJ, int CPR>
__device__ __forceinline__ void mma_stage(const uint4* as, const uint4* ws, int ra, int rb, int half,
                                          f32x16_t (&acc)[TI][TJ]) {
  bf16x8_t af[2][TI], bfr[2][TJ];
  auto load = [&](int s, int b) {
    const int kc = 2 * s + half;
#pragma unroll
    for (int i = 0; i < TI; ++i) af[b][i] = __builtin_bit_cast(bf16x8_t, as[swz<CPR>(ra + 32 * i, kc)]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) bfr[b][j] = __builtin_bit_cast(bf16x8_t, ws[swz<CPR>(rb + 32 * j, kc)]);
  };
  load(0, 0);
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    if (s + 1 < BK / 16) load(s + 1, (s + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s & 1][j], af[s & 1][i], acc[i][j], 0, 0, 0);
  }
}

// mma_stage with the next tile's loads spread over its first MFMAs: load l
// (of LOADS) is issued right after MFMA (l * SPREAD) / LOADS.  Issued
// together after the barrier, a tile's loads hold a wave at its issue for as
// long as the CU's memory pipeline takes to accept them (about 500 cycles for
// 32 KB, measured), with no MFMA running; between the MFMAs that time
// overlaps the matrix work.
template <int BK, int TI, int TJ, int CPR, int LOADS, int SPREAD, typename Issue>
__device__ __forceinline__ void mma_stage_il(const uint4* as, const uint4* ws, int ra, int rb, int half,
                                             f32x16_t (&acc)[TI][TJ], Issue issue_one) {
  static_assert(SPREAD <= (BK / 16) * TI * TJ, "loads spread over more MFMAs than the stage has");
  bf16x8_t af[2][TI], bfr[2][TJ];
  auto load = [&](int s, int b) {
    const int kc = 2 * s + half;
#pragma unroll
    for (int i = 0; i < TI; ++i) af[b][i] = __builtin_bit_cast(bf16x8_t, as[swz<CPR>(ra + 32 * i, kc)]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) bfr[b][j] = __builtin_bit_cast(bf16x8_t, ws[swz<CPR>(rb + 32 * j, kc)]);
  };
  load(0, 0);
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    if (s + 1 < BK / 16) load(s + 1, (s + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s & 1][j], af[s & 1][i], acc[i][j], 0, 0, 0);
        const int mi = (s * TI + i) * TJ + j;
#pragma unroll
        for (int l = 0; l < LOADS; ++l)
          if ((l * SPREAD) / LOADS == mi) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(l);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
  }
}

// One k-step of a wave's TI x TJ block of 32x32 tiles (fragments af, bfr)
// with the next step's TI + TJ fragment reads and NL tile loads placed
// between its MFMAs.  With a 128x128 wave tile (16 MFMAs a step) read r
// follows MFMA r, so the reads go out in the first half of the step and land
// under the second; with fewer MFMAs all reads follow the first MFMA.  Load l
// follows MFMA (l * MFMAs) / NL + (MFMAs / NL - 1), i.e. the last MFMA of its
// share.  The scheduling fences keep that order: the
// compiler waits for every outstanding LDS read once a direct-to-LDS load is
// in flight, so a read issued just before an MFMA that needs an older one
// would be waited for too.
template <int TI, int TJ, int NL, typename Read, typename Load>
__device__ __forceinline__ void mma_step_pipe(const bf16x8_t (&af)[TI], const bf16x8_t (&bfr)[TJ],
                                              f32x16_t (&acc)[TI][TJ], Read read_one, Load load_one) {
  constexpr int NR = TI + TJ, MF = TI * TJ;
  constexpr bool SPREAD_READS = MF >= 2 * NR;
  static_assert(NL <= 2 * MF, "loads fit between the step's MFMAs");
  constexpr int LOFF = NL > 0 && MF / NL > 1 ? MF / NL - 1 : 0;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int mi = i * TJ + j;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (SPREAD_READS) {
        if (mi < NR) {
          read_one(mi);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else if (mi == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) read_one(r);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int l = 0; l < NL; ++l)
        if ((l * MF) / NL + LOFF == mi) {
          load_one(l);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int EPI, int BM, int BN, int BK, int STAGES>
__global__ __launch_bounds__(kGemmThreads, (STAGES * (BM + BN) * BK * 2 <= 80 * 1024) ? 2 : 1)
void gemm_bf16_dtl_kernel(GemmArgs g) {
  constexpr int CPR = BK / 8;                          // 16-byte chunks per tile row
  constexpr int CHUNKS_A = BM * CPR, CHUNKS_B = BN * CPR;
  constexpr int LOADS_A = CHUNKS_A / kGemmThreads;     // direct-to-LDS loads per thread per k-tile
  constexpr int LOADS_B = CHUNKS_B / kGemmThreads;
  constexpr int LOADS = LOADS_A + LOADS_B;
  constexpr int TI = BM / 64, TJ = BN / 64;            // 32x32 blocks per wave
  static_assert(LOADS_A * kGemmThreads == CHUNKS_A && LOADS_B * kGemmThreads == CHUNKS_B, "tile/threads");
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.Nout + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  if (tile_empty(g, m0, BM)) return;

  __shared__ uint4 lds[STAGES][CHUNKS_A + CHUNKS_B];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int half = lane >> 5, col = lane & 31;
  const int K = g.K;
  // 64-bit tile bases; the per-thread offsets inside a tile stay 32-bit
  // (at most BM rows of K <= 2^22 elements)
  const bf16_t* A = static_cast<const bf16_t*>(g.a) + static_cast<size_t>(m0) * K;
  const bf16_t* W = static_cast<const bf16_t*>(g.w) + static_cast<size_t>(n0) * K;

  // load i of this thread fills LDS chunk c = (il*4 + wid)*64 + lane of its
  // operand (il = i for A, i - LOADS_A for W); it fetches the element chunk
  // that the swizzle maps there
  int goff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int il = i < LOADS_A ? i : i - LOADS_A;
    const int c = (il * 4 + wid) * 64 + lane;
    const int row = c / CPR;
    const int kc = swz_kc<CPR>(row, c % CPR);   // the XOR key is its own inverse
    if (i < LOADS_A) goff[i] = (min(m0 + row, g.M - 1) - m0) * K + kc * 8;
    else goff[i] = (min(n0 + row, g.Nout - 1) - n0) * K + kc * 8;
  }
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const bf16_t* src = (i < LOADS_A ? A : W) + goff[i] + kt * BK;
      const int il = i < LOADS_A ? i : i - LOADS_A;
      uint4* dst = &lds[stage][(i < LOADS_A ? 0 : CHUNKS_A) + (il * 4 + wid) * 64];
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)(dst), 16, 0, 0);
    }
  };

  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};

  const int ra = wm * (BM / 2) + col;
  const int rb = wn * (BN / 2) + col;

  const int nk = K / BK;
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < nk) issue(p, p);
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's chunks of tile kt have landed in LDS (tiles issued after
    // it may still be in flight) ...
    const int ahead = min(STAGES - 2, nk - 1 - kt);
    if constexpr (STAGES >= 4) {
      if (ahead >= 2) wait_vmcnt<2 * LOADS>();
      else if (ahead == 1) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
    } else if constexpr (STAGES == 3) {
      if (ahead >= 1) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    // ... and everybody's: a plain s_barrier, without the memory fence of
    // __syncthreads() that would also drain the loads still in flight
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    const uint4* as = lds[kt % STAGES];
    const uint4* ws = as + CHUNKS_A;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int kc = 2 * s + half;
      bf16x8_t af[TI], bfr[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) af[i] = __builtin_bit_cast(bf16x8_t, as[swz<CPR>(ra + 32 * i, kc)]);
#pragma unroll
      for (int j = 0; j < TJ; ++j) bfr[j] = __builtin_bit_cast(bf16x8_t, ws[swz<CPR>(rb + 32 * j, kc)]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  __syncthreads();   // every wave is done with the LDS stages
  int* tab = reinterpret_cast<int*>(&lds[0][0]);
  fill_row_table<EPI, BM>(g, m0, tab);
  __syncthreads();
  // staging after the row table
  static_assert(2 * BM * 4 + epi_stage_bytes<BM, BN, BM / 2>() <= sizeof(lds), "epilogue staging fits the LDS");
  tile_epilogue<EPI, BM, BN, TI, TJ, BM / 2, BN / 2, kGemmThreads>(
      g, acc, m0, n0, wm, wn, half, col, tab, reinterpret_cast<float*>(reinterpret_cast<char*>(&lds[0][0]) + 2 * BM * 4),
      true);
}

// ---------------------------------------------------------------------------
// In-workgroup split-K for outputs too small to put two workgroups on every
// CU: 8 waves in two groups of 4; group g multiplies k-tiles g, g+2, g+4, ...
// of the same 128x128 output tile with its own LDS stages, so each SIMD runs
// two waves; group 1 hands its accumulators to group 0 through LDS and group
// 0 adds them (fixed order) and runs the epilogue.
// ---------------------------------------------------------------------------

constexpr int kKs2Threads = 2 * kGemmThreads;

template <int EPI, int BK, int STAGES>
__global__ __launch_bounds__(kKs2Threads, 1) void gemm_bf16_dtl_ks2_kernel(GemmArgs g) {
  constexpr int BM = 128, BN = 128;
  constexpr int CPR = BK / 8;
  constexpr int CHUNKS_A = BM * CPR, CHUNKS_B = BN * CPR;
  constexpr int LOADS_A = CHUNKS_A / kGemmThreads;
  constexpr int LOADS_B = CHUNKS_B / kGemmThreads;
  constexpr int LOADS = LOADS_A + LOADS_B;
  constexpr int TI = 2, TJ = 2;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.Nout + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  if (tile_empty(g, m0, BM)) return;

  __shared__ uint4 lds[2][STAGES][CHUNKS_A + CHUNKS_B];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int grp = wid >> 2, gw = wid & 3;
  const int wm = gw >> 1, wn = gw & 1;
  const int half = lane >> 5, col = lane & 31;
  const int K = g.K;
  // 64-bit tile bases; the per-thread offsets inside a tile stay 32-bit
  // (at most BM rows of K <= 2^22 elements)
  const bf16_t* A = static_cast<const bf16_t*>(g.a) + static_cast<size_t>(m0) * K;
  const bf16_t* W = static_cast<const bf16_t*>(g.w) + static_cast<size_t>(n0) * K;

  int goff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int il = i < LOADS_A ? i : i - LOADS_A;
    const int c = (il * 4 + gw) * 64 + lane;
    const int row = c / CPR;
    const int kc = swz_kc<CPR>(row, c % CPR);
    if (i < LOADS_A) goff[i] = (min(m0 + row, g.M - 1) - m0) * K + kc * 8;
    else goff[i] = (min(n0 + row, g.Nout - 1) - n0) * K + kc * 8;
  }
  const int nk = K / BK;
  const int iters = (nk + 1) / 2;
  // iteration it of group grp multiplies k-tile 2*it + grp
  auto issue = [&](int it, int stage) {
    const int kt = 2 * it + grp;
    if (kt >= nk) return;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const bf16_t* src = (i < LOADS_A ? A : W) + goff[i] + kt * BK;
      const int il = i < LOADS_A ? i : i - LOADS_A;
      uint4* dst = &lds[grp][stage][(i < LOADS_A ? 0 : CHUNKS_A) + (il * 4 + gw) * 64];
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)(dst), 16, 0, 0);
    }
  };

  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};

  const int ra = wm * (BM / 2) + col;
  const int rb = wn * (BN / 2) + col;
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < iters) issue(p, p);
  for (int it = 0; it < iters; ++it) {
    // the counts of loads in flight differ between the groups only at the
    // very end (odd nk), where both wait for everything
    const int ahead = min(STAGES - 2, iters - 1 - it);
    if constexpr (STAGES == 3) {
      if (ahead >= 1 && 2 * (it + 1) + 1 < nk) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (it + STAGES - 1 < iters) issue(it + STAGES - 1, (it + STAGES - 1) % STAGES);
    if (2 * it + grp < nk) {
      const uint4* as = lds[grp][it % STAGES];
      const uint4* ws = as + CHUNKS_A;
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const int kc = 2 * s + half;
        bf16x8_t af[TI], bfr[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) af[i] = __builtin_bit_cast(bf16x8_t, as[swz<CPR>(ra + 32 * i, kc)]);
#pragma unroll
        for (int j = 0; j < TJ; ++j) bfr[j] = __builtin_bit_cast(bf16x8_t, ws[swz<CPR>(rb + 32 * j, kc)]);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
    }
  }

  __syncthreads();   // both groups are done with their LDS stages
  float* xch = reinterpret_cast<float*>(&lds[0][0][0]);                 // 64 KB: group 1's partials
  int* tab = reinterpret_cast<int*>(&lds[1][0][0]);                     // row table past them
  static_assert(sizeof(lds[0]) >= 4 * 64 * 64 * 4 && sizeof(lds[1]) >= 2 * 128 * 4, "LDS budget");
  if (grp == 1) {
    float* dst = xch + static_cast<size_t>(gw) * 64 * 64 + lane;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[((i * TJ + j) * 16 + v) * 64] = acc[i][j][v];
  } else {
    fill_row_table<EPI, BM>(g, m0, tab);
  }
  __syncthreads();
  if (grp == 0) {
    const float* src = xch + static_cast<size_t>(gw) * 64 * 64 + lane;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] += src[((i * TJ + j) * 16 + v) * 64];
  }
  __syncthreads();   // the exchange area is read; it now stages the epilogue (both groups store)
  static_assert(epi_stage_bytes<BM, BN, BM / 2>() <= sizeof(lds[0]), "epilogue staging fits the exchange area");
  tile_epilogue<EPI, BM, BN, TI, TJ, BM / 2, BN / 2, kKs2Threads>(g, acc, m0, n0, wm, wn, half, col, tab, xch,
                                                                  grp == 0);
}

// ---------------------------------------------------------------------------
// Work-balanced bf16 GEMM over the refreshed rows.
//
// The number of refreshed rows exists only on the device (k_eff), so the grid
// is sized for the most rows and every workgroup derives the work from k_eff:
// T active output tiles (row tiles of each episode's k_eff rows x column
// tiles).  With P workgroups resident at once, the first floor(T/P)*P tiles go
// one per workgroup; the r remaining tiles (the last, partly empty round) are
// split along K into S equal ranges, S chosen on the device from a cost model
// (rounds of the r*S pieces x (fixed piece cost + K/S)) and the workgroups
// the grid has to spare, so a small T, or a k_eff far below the rows the grid
// was sized for, still fills the CUs.  All pieces of one split index walk the same K range at the same
// time, so neighbouring tiles keep sharing operand lines in L2.  The last
// piece of a tile to finish (per-tile arrival counter) adds the S partial
// accumulators in split order -- independent of arrival order, so results are
// reproducible -- and runs the epilogue.  No workgroup ever waits for another.
// ---------------------------------------------------------------------------

#ifndef WAMC_SK_MIN_ITERS
#define WAMC_SK_MIN_ITERS 8
#endif
#ifndef WAMC_GEMM_SK
#define WAMC_GEMM_SK 1
#endif
#ifndef WAMC_SK_MAX_SPLIT
#define WAMC_SK_MAX_SPLIT 8
#endif
constexpr int kSkMinIters = WAMC_SK_MIN_ITERS;   // fewest k-tiles per split range
constexpr int kSkMaxSplit = WAMC_SK_MAX_SPLIT;   // most pieces per tile
#ifndef WAMC_SK_SLOT_ROUNDS
#define WAMC_SK_SLOT_ROUNDS 2
#endif
constexpr int kSkSlotRounds = WAMC_SK_SLOT_ROUNDS;   // partial-tile slots, in resident workgroups
#ifndef WAMC_SK_PIECE_COST
#define WAMC_SK_PIECE_COST 16
#endif
// fixed cost of one piece (pipeline fill, partial store, arrival, fix-up), in k-tiles
constexpr int kSkPieceCost = WAMC_SK_PIECE_COST;
// k-tiles from which the launch grid makes room for a split tail
#ifndef WAMC_SK_LONG_K
#define WAMC_SK_LONG_K 64
#endif
constexpr int kSkLongK = WAMC_SK_LONG_K;

// Pieces per tile for r tail tiles of nk k-tiles each, P resident
// workgroups and room for `room` pieces: S minimises (rounds of r*S pieces)
// x (piece overhead + nk/S k-tiles), each piece >= kSkMinIters k-tiles.  The
// host sizes the grid with it and the kernel re-derives it from k_eff.
__host__ __device__ inline int sk_split(int r, int nk, int P, int room) {
  if (r <= 0) return 1;
  int smax = nk / kSkMinIters;
  if (smax > kSkMaxSplit) smax = kSkMaxSplit;
  if (smax > room / r) smax = room / r;
  int S = 1;
  float best = static_cast<float>((r + P - 1) / P) * static_cast<float>(kSkPieceCost + nk);
  for (int c = 2; c <= smax; ++c) {
    const float cost = static_cast<float>((r * c + P - 1) / P) *
                       (static_cast<float>(kSkPieceCost) + static_cast<float>(nk) / static_cast<float>(c));
    if (cost < best) {
      best = cost;
      S = c;
    }
  }
  return S;
}

// Pieces per 256x256 tile of the plane split when the host leaves the count
// to the device (g.parts = -Smax): as many as keep the pieces within one
// workgroup per CU for the tiles of the k_eff rows, at most Smax.  The
// pieces kernel and the reduction both derive it from the same k_eff.
__device__ __forceinline__ int planes_split(const GemmArgs& g) {
  if (g.parts > 0) return g.parts;
  const int B = g.M / g.rows_cap;
  int tm = 0;
  for (int b = 0; b < B; ++b) tm += (rows_of(g.k_eff, b, g.rows_cap) + 255) / 256;
  const int tiles = tm * ((g.Nout + 255) / 256);
  return tiles > 0 ? max(1, min(-g.parts, 256 / tiles)) : 1;
}

struct SkTile {
  int m0, mend, n0;   // first row, end of the episode's valid rows, first column
};

// Active tile t (grouped order: 8 row tiles per column sweep) -> its rows/columns.
template <int BM, int BN>
__device__ __forceinline__ SkTile sk_tile(const GemmArgs& g, int t, int tiles_m, int tiles_n) {
  constexpr int GM = 8;
  const int group = t / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = t - group * GM * tiles_n;
  int tm = first_m + in_group % gsize;
  SkTile r{0, 0, (in_group / gsize) * BN};
  const int B = g.M / g.rows_cap;
  for (int b = 0; b < B; ++b) {
    const int rows = rows_of(g.k_eff, b, g.rows_cap);
    const int rt = (rows + BM - 1) / BM;
    if (tm < rt) {
      r.m0 = b * g.rows_cap + tm * BM;
      r.mend = b * g.rows_cap + rows;
      break;
    }
    tm -= rt;
  }
  return r;
}

// Resident workgroups of a configuration: two per CU when they fit (4 waves,
// <= 80 KiB LDS), else one.
#ifndef WAMC_SK_MAX_PER_CU
#define WAMC_SK_MAX_PER_CU 2
#endif
#ifndef WAMC_SK_GRID_ROUNDS
#define WAMC_SK_GRID_ROUNDS 3
#endif
// 256x256 tiles: 1 = fragment reads pipelined one k-step ahead across the
// barrier (mma_step_pipe); 0 = two k-steps' reads after each barrier
#ifndef WAMC_SK_IL_PIPE
#define WAMC_SK_IL_PIPE 1
#endif
constexpr bool kIlPipe = WAMC_SK_IL_PIPE != 0;
// the same loop for the 4-wave 128-row tiles of the work-balanced kernel
#ifndef WAMC_SK_PIPE
#define WAMC_SK_PIPE 0
#endif
constexpr bool kSkPipe = WAMC_SK_PIPE != 0;

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN>
struct SkConfig {
  static constexpr int kThreads = 64 * WGM * WGN;
  static constexpr int kLds = STAGES * (BM + BN) * BK * 2;
  // resident workgroups per CU: as many 4-wave workgroups as the LDS holds
  // (at most WAMC_SK_MAX_PER_CU); one for the 8-wave tiles
  static constexpr int kPerCu = kThreads == 256 ? (160 * 1024 / kLds < WAMC_SK_MAX_PER_CU ? 160 * 1024 / kLds
                                                                                          : WAMC_SK_MAX_PER_CU)
                                                : 1;
  static constexpr int kP = 256 * kPerCu;
  static constexpr size_t kTileBytes = static_cast<size_t>(BM) * BN * 4;
  static constexpr bool kIl = BM == 256 && BN == 256 && kThreads == 256 && STAGES == 2;
};

template <int EPI, int BM, int BN, int BK, int STAGES, int WGM, int WGN>
__global__ __launch_bounds__((SkConfig<BM, BN, BK, STAGES, WGM, WGN>::kThreads),
                             (SkConfig<BM, BN, BK, STAGES, WGM, WGN>::kPerCu))
void gemm_bf16_sk_kernel(GemmArgs g) {
  using Cfg = SkConfig<BM, BN, BK, STAGES, WGM, WGN>;
  constexpr int NT = Cfg::kThreads, NW = NT / 64;
  constexpr int CPR = BK / 8;
  constexpr int CHUNKS_A = BM * CPR, CHUNKS_B = BN * CPR;
  constexpr int LOADS_A = CHUNKS_A / NT;
  constexpr int LOADS_B = CHUNKS_B / NT;
  constexpr int LOADS = LOADS_A + LOADS_B;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;         // wave tile
  constexpr int TI = WTM / 32, TJ = WTN / 32;
  static_assert(LOADS_A * NT == CHUNKS_A && LOADS_B * NT == CHUNKS_B, "tile/threads");
  static_assert(TI * 32 == WTM && TJ * 32 == WTN, "wave tile");
  // one 4-wave workgroup per CU on 256x256 tiles (128x128 per wave): the next
  // tile's loads go between the MFMAs of the first half of each stage
  constexpr bool IL = Cfg::kIl;
  // the cross-barrier pipelined loop (256x256 tiles; 128x128 and 128x192 as a build option)
  constexpr bool PIPE = IL ? kIlPipe : (kSkPipe && STAGES == 2 && BK == 64 && NT == 256);

  const int B = g.M / g.rows_cap;
  int tiles_m = 0;
  for (int b = 0; b < B; ++b) tiles_m += (rows_of(g.k_eff, b, g.rows_cap) + BM - 1) / BM;
  const int tiles_n = (g.Nout + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  constexpr int P = Cfg::kP;
  const int slots = static_cast<int>(min(g.sk_partial_bytes / Cfg::kTileBytes, static_cast<size_t>(kSkSlotRounds * P)));
  // planes (wide tiles only): every tile is cut into g.parts K-pieces that
  // store raw f32 accumulators to plane [piece][M][Nout]; a second kernel sums
  // the planes in piece order and applies the epilogue
  const bool planes = IL && (g.parts > 1 || g.parts < 0);
  const int ndp = planes ? 0 : (tiles / P) * P;   // tiles done one per workgroup
  const int r = tiles - ndp;                       // tail tiles, split along K
  const int nk = g.K / BK;
  // Work items: the ndp tiles done whole, then the r*S pieces of the split
  // tail.  Workgroup h takes items h, h + G, h + 2G, ... (G = the grid, a
  // multiple of the 8 XCDs: an item runs on the XCD its remapped index
  // belongs to).  The pieces fit the grid's spare workgroups and the partial
  // slots.
  const int G = static_cast<int>(gridDim.x);
  // (the wide tiles' grid of one workgroup per CU leaves room to split a few
  // dozen short-K tiles, whose partial tiles cost more than the split saves)
  const int S = planes ? planes_split(g) : IL && nk < kSkLongK ? 1 : sk_split(r, nk, P, min(max(G - ndp, 0), slots));
  const int W = ndp + r * S;

  // one LDS object only: a second __shared__ variable makes the compiler wait
  // for the tile loads in flight before every LDS read (it cannot tell the
  // objects apart from the direct-to-LDS writes)
  __shared__ uint4 lds[STAGES][CHUNKS_A + CHUNKS_B];
  int* s_last = reinterpret_cast<int*>(&lds[STAGES - 1][CHUNKS_A + CHUNKS_B - 1]);   // clear of the row table

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int half = lane >> 5, col = lane & 31;
  const bf16_t* A = static_cast<const bf16_t*>(g.a);
  const bf16_t* Wt = static_cast<const bf16_t*>(g.w);
  const int K = g.K;

  for (int w = blockIdx.x; w < W; w += G) {
    // this item: tile tl, k-tiles [kk0, kk1); a piece of a split tile when split
    const bool split = w >= ndp && S > 1;
    SkTile tl;
    int kk0 = 0, kk1 = nk, tt = 0, u = 0, sp = 0;
    if (w < ndp) {
      tl = sk_tile<BM, BN>(g, xcd_remap(w, ndp), tiles_m, tiles_n);
    } else {
      u = xcd_remap(w - ndp, r * S);
      if (planes) {
        // consecutive items (one XCD) share a K range and neighbouring tiles' panels
        sp = u / r;
        tt = u - sp * r;
      } else {
        tt = u / S;
        sp = u - tt * S;   // split index
      }
      tl = sk_tile<BM, BN>(g, ndp + tt, tiles_m, tiles_n);
      kk0 = sp * nk / S;
      kk1 = (sp + 1) * nk / S;
    }

    int goff[IL ? 1 : LOADS];
    if constexpr (!IL) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int il = i < LOADS_A ? i : i - LOADS_A;
        const int c = (il * NW + wid) * 64 + lane;
        const int row = c / CPR;
        const int kc = swz_kc<CPR>(row, c % CPR);
        if (i < LOADS_A) goff[i] = (min(tl.m0 + row, g.M - 1) - tl.m0) * K + kc * 8 + kk0 * BK;
        else goff[i] = (min(tl.n0 + row, g.Nout - 1) - tl.n0) * K + kc * 8 + kk0 * BK;
      }
    }
    // IL: load il of thread tid covers tile row r0 + 32 il at element column kcol
    static_assert(!IL || (CPR == 8 && NT / CPR == 32), "interleaved loads: 32 rows per load");
    const int r0 = tid / CPR, kcol = swz_kc<CPR>(r0, tid % CPR) * 8;
    const int mlim = g.M - 1 - tl.m0, nlim = g.Nout - 1 - tl.n0;
    // 64-bit tile bases; the per-thread offsets inside a tile stay 32-bit
    // (at most BM rows of K <= 2^22 elements)
    const bf16_t* At = A + static_cast<size_t>(tl.m0) * K;
    const bf16_t* Wtt = Wt + static_cast<size_t>(tl.n0) * K;
    auto issue = [&](int kt, int stage) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int il = i < LOADS_A ? i : i - LOADS_A;
        int off;
        if constexpr (IL) off = min(r0 + 32 * il, i < LOADS_A ? mlim : nlim) * K + kcol + (kk0 + kt) * BK;
        else off = goff[i] + kt * BK;
        const bf16_t* src = (i < LOADS_A ? At : Wtt) + off;
        uint4* dst = &lds[stage][(i < LOADS_A ? 0 : CHUNKS_A) + (il * NW + wid) * 64];
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)(dst), 16, 0, 0);
      }
    };

    f32x16_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};

    const int ra = wm * WTM + col;
    const int rb = wn * WTN + col;
    const int n = kk1 - kk0;
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (p < n) issue(p, p);
    if constexpr (PIPE) {
      // Fragment reads one k-step ahead of the MFMAs, across the barrier.
      // Per tile q (stage q&1): steps 0-2 each read the next step's fragments
      // between their MFMAs; then every wave waits for its loads of tile q+1
      // and its last reads of stage q&1, and one barrier makes both hold for
      // the workgroup; step 3 then reads step 0 of tile q+1 from the other
      // stage and starts tile q+2's loads into stage q&1.  The 256x256 tiles
      // send a tile's loads out in two halves, during step 3 of the tile
      // before and step 0 of their own, three to four k-steps before the
      // barrier that needs them, with clamped tile indices past the last tile
      // (the last tile loaded again into a stage no later step reads: no
      // branch among the MFMAs); the 128x128 tiles send all of them during
      // step 3, four k-steps ahead.
      static_assert(STAGES == 2 && BK / 16 == 4 && LOADS % 2 == 0, "pipelined loop: two stages of four k-steps");
      constexpr int LH = IL ? LOADS / 2 : LOADS;   // loads per issue window
      bf16x8_t af0[TI], bf0[TJ], af1[TI], bf1[TJ];
      // read r of step s (stage `st`) into (naf, nbf), in the order the MFMAs use them
      auto reader = [&](bf16x8_t(&naf)[TI], bf16x8_t(&nbf)[TJ], const uint4* st, int s) {
        const uint4* wst = st + CHUNKS_A;
        const int kc = 2 * s + half;
        return [&naf, &nbf, st, wst, kc, ra, rb](int r) {
          if (r == 0) naf[0] = __builtin_bit_cast(bf16x8_t, st[swz<CPR>(ra, kc)]);
          else if (r <= TJ) nbf[r - 1] = __builtin_bit_cast(bf16x8_t, wst[swz<CPR>(rb + 32 * (r - 1), kc)]);
          else naf[r - TJ] = __builtin_bit_cast(bf16x8_t, st[swz<CPR>(ra + 32 * (r - TJ), kc)]);
        };
      };
      // load l of window h of tile `tile` into stage `stage`
      auto loader = [&](int tile, int stage, int h) {
        const int kb = kcol + (kk0 + tile) * BK;
        return [&, kb, tile, stage, h](int l) {
          const int i = h * LH + l;
          const int il = i < LOADS_A ? i : i - LOADS_A;
          int off;
          // IL: rows r0 + 32 il of the tile, clamped to the last valid row
          // (the swizzle key is the same for every il: 32 rows keep (row >> 1) & 7)
          if constexpr (IL) off = min(r0 + 32 * il, i < LOADS_A ? mlim : nlim) * K + kb;
          else off = goff[i] + tile * BK;
          const bf16_t* src = (i < LOADS_A ? At : Wtt) + off;
          uint4* dst = &lds[stage][(i < LOADS_A ? 0 : CHUNKS_A) + (il * NW + wid) * 64];
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)(dst), 16, 0, 0);
        };
      };
      auto no_load = [](int) {};
      if (n > 0) {
        wait_vmcnt<0>();   // tile 0 has landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        {
          auto rd = reader(af0, bf0, lds[0], 0);
#pragma unroll
          for (int r = 0; r < TI + TJ; ++r) rd(r);
          if (IL || n > 1) {
            auto ld = loader(min(1, n - 1), 1, 0);
#pragma unroll
            for (int l = 0; l < LH; ++l) ld(l);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        for (int q = 0; q < n; ++q) {
          const uint4* cur = lds[q & 1];
          const uint4* nxt = lds[(q + 1) & 1];
          if constexpr (IL)
            mma_step_pipe<TI, TJ, LH>(af0, bf0, acc, reader(af1, bf1, cur, 1),
                                      loader(min(q + 1, n - 1), (q + 1) & 1, 1));
          else
            mma_step_pipe<TI, TJ, 0>(af0, bf0, acc, reader(af1, bf1, cur, 1), no_load);
          mma_step_pipe<TI, TJ, 0>(af1, bf1, acc, reader(af0, bf0, cur, 2), no_load);
          mma_step_pipe<TI, TJ, 0>(af0, bf0, acc, reader(af1, bf1, cur, 3), no_load);
          __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile q+1 and reads of stage q&1 are done
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          if (IL || q + 2 < n)
            mma_step_pipe<TI, TJ, LH>(af1, bf1, acc, reader(af0, bf0, nxt, 0), loader(min(q + 2, n - 1), q & 1, 0));
          else
            mma_step_pipe<TI, TJ, 0>(af1, bf1, acc, reader(af0, bf0, nxt, 0), no_load);
        }
      }
      wait_vmcnt<0>();   // the trailing loads land before the LDS is used again
    } else if constexpr (IL) {
      static_assert(STAGES == 2, "interleaved loads: two stages");
      for (int q = 0; q < n; ++q) {
        wait_vmcnt<0>();   // tile q has landed
        __builtin_amdgcn_s_barrier();
        // tile q + 1 into the other stage; past the last tile the last one is
        // read again into the stage no later step reads (no branch among the MFMAs)
        const int nt = min(q + 1, n - 1), ns = (q + 1) & 1;
        const uint4* as = lds[q & 1];
        const int kb = kcol + (kk0 + nt) * BK;
        mma_stage_il<BK, TI, TJ, CPR, LOADS, (BK / 16) * TI * TJ / 2>(
            as, as + CHUNKS_A, ra, rb, half, acc, [&](int i) {
              // rows r0 + 32 il of the tile, clamped to the last valid row; the
              // swizzle key is the same for every il (32 rows keep (row >> 1) & 7)
              const int il = i < LOADS_A ? i : i - LOADS_A;
              const int off = min(r0 + 32 * il, i < LOADS_A ? mlim : nlim) * K + kb;
              const bf16_t* src = (i < LOADS_A ? At : Wtt) + off;
              uint4* dst = &lds[ns][(i < LOADS_A ? 0 : CHUNKS_A) + (il * NW + wid) * 64];
              __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)(dst), 16, 0, 0);
            });
      }
      wait_vmcnt<0>();   // the last tile's extra loads land before the LDS is used again
    } else {
      for (int q = 0; q < n; ++q) {
        // tile q has landed once at most (tiles issued after it) x LOADS loads remain
        wait_tiles_ahead<LOADS, STAGES - 2>(min(STAGES - 2, n - 1 - q));
        __builtin_amdgcn_s_barrier();
        if (q + STAGES - 1 < n) issue(q + STAGES - 1, (q + STAGES - 1) % STAGES);
        const uint4* as = lds[q % STAGES];
        mma_stage<BK, TI, TJ, CPR>(as, as + CHUNKS_A, ra, rb, half, acc);
      }
    }

    auto finish = [&]() {
      __syncthreads();   // every wave is done with the LDS stages
      int* tab = reinterpret_cast<int*>(&lds[0][0]);
      fill_row_table<EPI, BM, NT>(g, tl.m0, tab, tl.mend);
      __syncthreads();
      // staging after the row table, clear of the split flag at the end
      static_assert(2 * BM * 4 + epi_stage_bytes<BM, BN, WTM>() + 16 <= sizeof(lds), "epilogue staging fits the LDS");
      float* stage = reinterpret_cast<float*>(reinterpret_cast<char*>(&lds[0][0]) + 2 * BM * 4);
      if constexpr (IL) {
        // staged for every epilogue: it stores the accumulators to LDS straight
        // from their registers, where the direct one needs them all moved to
        // the vector registers the 128x128 wave tile has no room for
        tile_epilogue_staged<EPI, BM, BN, TI, TJ, WTM, WTN, NT>(g, acc, tl.n0, wm, wn, half, col, tab, stage, true);
      } else {
        tile_epilogue<EPI, BM, BN, TI, TJ, WTM, WTN, NT>(g, acc, tl.m0, tl.n0, wm, wn, half, col, tab, stage, true);
      }
    };
    if (!split) {
      finish();
    } else if (planes) {
      // lane (half, col) of block (i, j) holds row wm*WTM + 32i + col, columns
      // wn*WTN + 32j + 8gg + 4half + (0..3); valid rows and columns only
      float* plane = g.sk_partial + static_cast<size_t>(sp) * g.M * g.Nout;
      // The row and column checks are all taken before the first store and
      // kept in two registers: the kernel runs at its register limit, and a
      // bound reloaded from the spill area between the row blocks waited
      // (vmcnt) for every store issued before it.
      const int m0r = tl.m0 + wm * WTM + col, c0 = tl.n0 + wn * WTN + 4 * half;
      static_assert(TI + 4 * TJ <= 32, "row and column checks fit one register");
      unsigned ok = 0;
#pragma unroll
      for (int i = 0; i < TI; ++i) ok |= (m0r + 32 * i < tl.mend ? 1u : 0u) << i;
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) ok |= (c0 + 32 * j + 8 * gg < g.Nout ? 1u : 0u) << (TI + j * 4 + gg);
      // (a global pointer: through the asm statement a generic one would turn the stores into flat ones)
      gf32x4_t* prow = (gf32x4_t*)(plane + static_cast<size_t>(m0r) * g.Nout + c0);
      asm volatile("" : "+v"(ok), "+v"(prow));
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        if (!((ok >> i) & 1u)) continue;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg)
            if ((ok >> (TI + j * 4 + gg)) & 1u)
              prow[(static_cast<size_t>(32 * i) * g.Nout + 32 * j + 8 * gg) / 4] =
                  f32x4_v{acc[i][j][4 * gg], acc[i][j][4 * gg + 1], acc[i][j][4 * gg + 2], acc[i][j][4 * gg + 3]};
      }
    } else {
      // Partial tiles live in scratch slot u (piece u of the tail).  They are
      // written and read as relaxed system-scope atomics (sc0 sc1 accesses that go
      // to the coherence point and back), so no cache-wide write-back or
      // invalidate is needed between the workgroups of one tile.
      unsigned long long* part = reinterpret_cast<unsigned long long*>(g.sk_partial);
      const size_t own = static_cast<size_t>(u) * (BM * BN / 2);   // 8-byte words
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int v2 = 0; v2 < 8; ++v2) {
            const unsigned long long x = (static_cast<unsigned long long>(__float_as_uint(acc[i][j][2 * v2 + 1])) << 32) |
                                         __float_as_uint(acc[i][j][2 * v2]);
            __hip_atomic_store(part + own + static_cast<size_t>(((i * TJ + j) * 8 + v2) * NT + tid), x,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          }
      // the stores have reached the coherence point before the arrival is counted
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        int* cnt = &g.sk_counters[ndp + tt];
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        const int last = old == S - 1 ? 1 : 0;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);   // ready for the next launch
        *s_last = last;
      }
      __syncthreads();
      if (*s_last) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};
        for (int v = 0; v < S; ++v) {
          const unsigned long long* src = part + static_cast<size_t>(tt * S + v) * (BM * BN / 2);
#pragma unroll
          for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
              // one 32x32 block at a time keeps the loads' registers few
              unsigned long long p[8];
#pragma unroll
              for (int v2 = 0; v2 < 8; ++v2)
                p[v2] = __hip_atomic_load(src + static_cast<size_t>(((i * TJ + j) * 8 + v2) * NT + tid), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_SYSTEM);
#pragma unroll
              for (int v2 = 0; v2 < 8; ++v2) {
                acc[i][j][2 * v2] += __uint_as_float(static_cast<unsigned>(p[v2]));
                acc[i][j][2 * v2 + 1] += __uint_as_float(static_cast<unsigned>(p[v2] >> 32));
              }
            }
        }
        finish();
      }
    }
    __syncthreads();   // the next item's tile loads overwrite the LDS read above
  }
}

// ---------------------------------------------------------------------------
// Split-K pieces with a separate reduction (few output tiles)
//
// With a few hundred rows the projections have a few dozen 128x128 tiles, and
// a kernel that gives each tile one workgroup waits one load round trip per
// k-tile on a handful of CUs.  Here every 64x128 or 128x128 tile is cut
// along K into S pieces, one workgroup each, so the tiles x S workgroups fill
// the CUs; each
// piece stores its raw f32 accumulators to its own plane of the scratch,
// [S][M][Nout], valid rows only.  A second kernel sums the S planes of each
// element in piece order (so the result does not depend on which piece ran
// first) and applies the epilogue, spread over every CU.  Measured at
// d = 1536 with 70 to 1080 rows this beats both the one-tile-per-workgroup
// kernels and the work-balanced kernel's split, whose last piece reads all
// S partial tiles itself, one round trip to the coherence point per piece.
// ---------------------------------------------------------------------------
#ifndef WAMC_GEMM_PARTS
#define WAMC_GEMM_PARTS 1
#endif
#ifndef WAMC_PARTS_RESIDENT
#define WAMC_PARTS_RESIDENT 512
#endif
#ifndef WAMC_PARTS_MIN_ITERS
#define WAMC_PARTS_MIN_ITERS 6
#endif
#ifndef WAMC_PARTS_MAX_SPLIT
#define WAMC_PARTS_MAX_SPLIT 16
#endif
constexpr int kPartsBN = 128, kPartsBK = 64;
constexpr int kPartsTallRows = 384;   // rows from which a long-K split takes 128-row tiles
constexpr int kPartsResident = WAMC_PARTS_RESIDENT;   // two 4-wave workgroups (48 or 64 KiB LDS each) per CU
constexpr int kPartsMinIters = WAMC_PARTS_MIN_ITERS;  // fewest k-tiles per piece
constexpr int kPartsMaxSplit = WAMC_PARTS_MAX_SPLIT;

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN, 2) void gemm_bf16_parts_kernel(GemmArgs g) {
  constexpr int NT = 64 * WGM * WGN, NW = NT / 64;
  constexpr int CPR = BK / 8;
  constexpr int CHUNKS_A = BM * CPR, CHUNKS_B = BN * CPR;
  constexpr int LOADS_A = CHUNKS_A / NT;
  constexpr int LOADS_B = CHUNKS_B / NT;
  constexpr int LOADS = LOADS_A + LOADS_B;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TI = WTM / 32, TJ = WTN / 32;
  static_assert(LOADS_A * NT == CHUNKS_A && LOADS_B * NT == CHUNKS_B, "tile/threads");
  static_assert(TI * 32 == WTM && TJ * 32 == WTN, "wave tile");

  const int S = g.parts;
  const int B = g.M / g.rows_cap;
  int tiles_m = 0;
  for (int b = 0; b < B; ++b) tiles_m += (rows_of(g.k_eff, b, g.rows_cap) + BM - 1) / BM;
  const int tiles_n = (g.Nout + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int items = tiles * S;   // the grid is sized for rows_cap rows: the rest exit
  if (static_cast<int>(blockIdx.x) >= items) return;
  // item v = piece sp of tile t; consecutive items (one XCD) share a W panel and K range
  const int v = xcd_remap(blockIdx.x, items);
  const int sp = v / tiles;
  const SkTile tl = sk_tile<BM, BN>(g, v - sp * tiles, tiles_m, tiles_n);
  const int nk_all = g.K / BK;
  const int kk0 = sp * nk_all / S, n = (sp + 1) * nk_all / S - kk0;

  __shared__ uint4 lds[STAGES][CHUNKS_A + CHUNKS_B];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int half = lane >> 5, col = lane & 31;
  const int K = g.K;
  int goff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int il = i < LOADS_A ? i : i - LOADS_A;
    const int c = (il * NW + wid) * 64 + lane;
    const int row = c / CPR;
    const int kc = swz_kc<CPR>(row, c % CPR);
    if (i < LOADS_A) goff[i] = (min(tl.m0 + row, g.M - 1) - tl.m0) * K + kc * 8 + kk0 * BK;
    else goff[i] = (min(tl.n0 + row, g.Nout - 1) - tl.n0) * K + kc * 8 + kk0 * BK;
  }
  const bf16_t* At = static_cast<const bf16_t*>(g.a) + static_cast<size_t>(tl.m0) * K;
  const bf16_t* Wtt = static_cast<const bf16_t*>(g.w) + static_cast<size_t>(tl.n0) * K;
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const bf16_t* src = (i < LOADS_A ? At : Wtt) + goff[i] + kt * BK;
      const int il = i < LOADS_A ? i : i - LOADS_A;
      uint4* dst = &lds[stage][(i < LOADS_A ? 0 : CHUNKS_A) + (il * NW + wid) * 64];
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)(dst), 16, 0, 0);
    }
  };
  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};
  const int ra = wm * WTM + col, rb = wn * WTN + col;
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < n) issue(p, p);
  for (int q = 0; q < n; ++q) {
    wait_tiles_ahead<LOADS, STAGES - 2>(min(STAGES - 2, n - 1 - q));
    __builtin_amdgcn_s_barrier();
    if (q + STAGES - 1 < n) issue(q + STAGES - 1, (q + STAGES - 1) % STAGES);
    const uint4* as = lds[q % STAGES];
    mma_stage<BK, TI, TJ, CPR>(as, as + CHUNKS_A, ra, rb, half, acc);
  }
  // lane (half, col) of block (i, j) holds row wm*WTM + 32i + col, columns
  // wn*WTN + 32j + 8gg + 4half + (0..3) (the operands are issued W first)
  float* plane = g.sk_partial + static_cast<size_t>(sp) * g.M * g.Nout;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int m = tl.m0 + wm * WTM + 32 * i + col;
    if (m >= tl.mend) continue;
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int c = tl.n0 + wn * WTN + 32 * j + 8 * gg + 4 * half;
        if (c < g.Nout)
          *reinterpret_cast<float4*>(plane + static_cast<size_t>(m) * g.Nout + c) =
              make_float4(acc[i][j][4 * gg], acc[i][j][4 * gg + 1], acc[i][j][4 * gg + 2], acc[i][j][4 * gg + 3]);
      }
  }
}

// Sum of the S planes in piece order, then the epilogue of the tile kernels
// (v = acc + bias; act(v), or resid + gate * v as one fma), four columns a
// thread (Nout % 4 == 0, so a group lies in one of Q | K | V).
template <int EPI>
__global__ __launch_bounds__(256) void gemm_parts_epilogue_kernel(GemmArgs g) {
  const int S = planes_split(g);
  const int groups = g.Nout / 4;
  const long long total = static_cast<long long>(g.M) * groups;
  const size_t plane = static_cast<size_t>(g.M) * g.Nout;
  const bf16_t* bias = static_cast<const bf16_t*>(g.bias);
  const QkvDst qd = qkv_dst(g);
  for (long long q = blockIdx.x * 256LL + threadIdx.x; q < total; q += static_cast<long long>(gridDim.x) * 256) {
    const int m = static_cast<int>(q / groups);
    const int c = static_cast<int>(q - static_cast<long long>(m) * groups) * 4;
    const RowInfo ri = row_info(g, m);
    if (!ri.valid) continue;
    const float* src = g.sk_partial + static_cast<size_t>(m) * g.Nout + c;
    float4 a = *reinterpret_cast<const float4*>(src);
    // planes 1.. in batches of four whose loads are in flight together; the
    // additions stay in plane order
    int p = 1;
    for (; p + 4 <= S; p += 4) {
      float4 x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = *reinterpret_cast<const float4*>(src + (p + q) * plane);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a.x += x[q].x; a.y += x[q].y; a.z += x[q].z; a.w += x[q].w;
      }
    }
    for (; p < S; ++p) {
      const float4 x = *reinterpret_cast<const float4*>(src + p * plane);
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    }
    const uint2 bb = *reinterpret_cast<const uint2*>(bias + c);
    float y[4] = {a.x + __uint_as_float(bb.x << 16), a.y + __uint_as_float(bb.x & 0xffff0000u),
                  a.z + __uint_as_float(bb.y << 16), a.w + __uint_as_float(bb.y & 0xffff0000u)};
    if constexpr (EPI == EPI_RESID_OUT || EPI == EPI_RESID_DOWN || EPI == EPI_RESID_PLAIN) {
      uint2 gt = make_uint2(0x3f803f80u, 0x3f803f80u);   // 1.0 in bf16: ungated
      if constexpr (EPI != EPI_RESID_PLAIN) gt = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(g.gate) + c);
      const size_t o = static_cast<size_t>(m) * g.Nout + c;
      const float4 xin = *reinterpret_cast<const float4*>(g.resid_in + o);
      float4 xo;
      xo.x = fmaf(__uint_as_float(gt.x << 16), y[0], xin.x);
      xo.y = fmaf(__uint_as_float(gt.x & 0xffff0000u), y[1], xin.y);
      xo.z = fmaf(__uint_as_float(gt.y << 16), y[2], xin.z);
      xo.w = fmaf(__uint_as_float(gt.y & 0xffff0000u), y[3], xin.w);
      *reinterpret_cast<float4*>(g.resid_out + o) = xo;
    } else {
      if constexpr (EPI == EPI_GELU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = gelu_erf_fast(y[e]);
      }
      uint2 w;
      w.x = pack_bf16x2(y[0], y[1]);
      w.y = pack_bf16x2(y[2], y[3]);
      if constexpr (EPI == EPI_QKV || EPI == EPI_KV) {
        const int d = g.d_model;
        const int wr = c / d, cc = c - wr * d;
        const int which = wr + (EPI == EPI_KV ? 1 : 0);
        int r = m;
        if (which != 0) {
          const int tok = g.idx ? g.idx[static_cast<size_t>(ri.b) * g.n_tokens + ri.r] : ri.r;
          r = (tok >= 0 && tok < g.n_tokens) ? ri.b * g.n_tokens + tok : -1;
        }
        gbf16_t* dst = qkv_pick(qd, which);
        if (r >= 0) *reinterpret_cast<gu32x2_t*>(dst + static_cast<size_t>(r) * d + cc) = __builtin_bit_cast(u32x2_v, w);
      } else {
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.g_out) + static_cast<size_t>(m) * g.Nout + c) = w;
      }
    }
  }
}

// The reduction of a residual projection (Nout = d) fused with the
// LayerNorm that follows it: one wavefront per row (4 rows a block), lane
// chunks as in the row kernels, so the row's x is bitwise that of the
// reduction above and its h that of the LayerNorm kernel, and one launch
// replaces two.
template <int NC, int EPI, bool MOD>
__global__ __launch_bounds__(256) void gemm_parts_resid_ln_kernel(GemmArgs g) {
  static_assert(EPI == EPI_RESID_OUT || EPI == EPI_RESID_DOWN || EPI == EPI_RESID_PLAIN, "residual epilogues");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int m = blockIdx.x * 4 + wid;
  if (m >= g.M || !row_info(g, m).valid) return;
  const int d = g.Nout, S = planes_split(g);
  const size_t plane = static_cast<size_t>(g.M) * d;
  const float* src = g.sk_partial + static_cast<size_t>(m) * d;
  float v[NC][4];
  load_row<NC>(src, d, lane, v);
  // planes 1.. in pairs whose loads are in flight together, added in plane order
  int p = 1;
  for (; p + 2 <= S; p += 2) {
    float t[2][NC][4];
    load_row<NC>(src + p * plane, d, lane, t[0]);
    load_row<NC>(src + (p + 1) * plane, d, lane, t[1]);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[j][i] += t[q][j][i];
  }
  if (p < S) {
    float t[NC][4];
    load_row<NC>(src + p * plane, d, lane, t);
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[j][i] += t[j][i];
  }
  float bs[NC][4], gt[NC][4], xin[NC][4];
  load_row<NC>(static_cast<const bf16_t*>(g.bias), d, lane, bs);
  if constexpr (EPI != EPI_RESID_PLAIN) {
    load_row<NC>(static_cast<const bf16_t*>(g.gate), d, lane, gt);
  } else {
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) gt[j][i] = 1.0f;
  }
  load_row<NC>(g.resid_in + static_cast<size_t>(m) * d, d, lane, xin);
  RowMod<NC, bf16_t, MOD> md;
  md.load(static_cast<const bf16_t*>(g.ln_shift), static_cast<const bf16_t*>(g.ln_scale), d, lane);
  float* xo = g.resid_out + static_cast<size_t>(m) * d;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (j * 256 >= d) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[j][i] = fmaf(gt[j][i], v[j][i] + bs[j][i], xin[j][i]);
    const int c = lane * 4 + j * 256;
    if (c < d) *reinterpret_cast<float4*>(xo + c) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
  }
  float mean, rstd;
  row_stats(v, d, lane, g.ln_eps, mean, rstd);
  row_norm_store<NC, bf16_t, MOD>(v, d, lane, mean, rstd, md, static_cast<bf16_t*>(g.ln_out) + static_cast<size_t>(m) * d);
}

template <int EPI>
static void launch_parts_resid_ln(const GemmArgs& gp, int nc, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((gp.M + 3) / 4);
  const bool mod = gp.ln_shift != nullptr;
  WAMC_ROW_NC_DISPATCH(nc, if constexpr (NC > 0) {
    if (mod) launch(gemm_parts_resid_ln_kernel<NC, EPI, true>, grid, 256, 0, s, gp);
    else launch(gemm_parts_resid_ln_kernel<NC, EPI, false>, grid, 256, 0, s, gp);
  })
}

// Pieces per tile (S = 1: the path is not taken) and the tile height of the
// split-K path.  S is as large as keeps the tiles x S workgroups within one
// round of the resident workgroups, with at least kPartsMinIters k-tiles per
// piece and the S planes within the scratch.  Measured at d = 1536, 70 to
// 1080 rows: with a long K (the MLP down projection) any split pays, and from
// a few hundred rows on 128-row tiles, which read A and W half as often, beat
// 64-row ones (1080 rows: 55 against 69 us); with a short K a two-piece split
// loses to the in-workgroup split-K kernel (QKV at 280 rows: 24 against 20 us;
// the long-K down projection at 2458 rows: 94 against 86 us), so wherever that
// kernel would run the path takes three pieces or more, or two where the
// reduction also does the LayerNorm that follows (a launch of its own
// otherwise).
struct PartsPlan {
  int S, bm;
};
// whether the split-K reduction of this launch can do the LayerNorm after it
static bool parts_ln_fuses(GemmEpi epi, const GemmArgs& g) {
  const bool resid = epi == EPI_RESID_OUT || epi == EPI_RESID_DOWN || epi == EPI_RESID_PLAIN;
  return resid && g.ln_out != nullptr && g.Nout == g.d_model && row_chunks(g.d_model) > 0;
}
static PartsPlan parts_plan(GemmEpi epi, const GemmArgs& g, bool ks2_runs) {
  PartsPlan p{1, 64};
  if (!WAMC_GEMM_PARTS || !g.sk_partial || g.K % kPartsBK != 0 || g.Nout % 4 != 0) return p;
  const int nk = g.K / kPartsBK;
  const bool long_k = nk >= kSkLongK;
  p.bm = long_k && g.M >= kPartsTallRows ? 128 : 64;
  const long long tiles = static_cast<long long>(g.M / g.rows_cap) * ((g.rows_cap + p.bm - 1) / p.bm) *
                          ((g.Nout + kPartsBN - 1) / kPartsBN);
  const long long plane = static_cast<long long>(g.M) * g.Nout * 4;
  long long S = std::min<long long>(kPartsResident / tiles, nk / kPartsMinIters);
  S = std::min<long long>(S, kPartsMaxSplit);
  S = std::min<long long>(S, static_cast<long long>(g.sk_partial_bytes) / plane);
  p.S = S >= ((long_k && !ks2_runs) || parts_ln_fuses(epi, g) ? 2 : 3) ? static_cast<int>(S) : 1;
  return p;
}

#ifndef WAMC_GEMM_BIG
#define WAMC_GEMM_BIG 1
#endif
// 256x256 tiles (8 waves, one workgroup per CU) for the work-balanced path
// when there are at least two full rounds of them (measured: 36-39 % of peak
// against 33-36 % for 128x128 tiles at 16k rows; slower at 2.5-4.7k rows,
// where the tile count leaves a large ragged round)
constexpr bool kGemmBig = WAMC_GEMM_BIG != 0;
#ifndef WAMC_SK_BK
#define WAMC_SK_BK 64
#endif
#ifndef WAMC_SK_STAGES
#define WAMC_SK_STAGES 2
#endif
#ifndef WAMC_SK_BM
#define WAMC_SK_BM 128
#endif

#ifndef WAMC_SK_BN
#define WAMC_SK_BN 128
#endif
#ifndef WAMC_SK_WGM
#define WAMC_SK_WGM 2
#endif
#ifndef WAMC_SK_WGN
#define WAMC_SK_WGN 2
#endif
// (measured on the d=1536 shapes: 128x256 / 256x128 wave tiles; 256x128 and
// 128x256 tiles on 8 waves with BK 64 and 2 or 3 stages or BK 32 and 4;
// BK 32 with 3 to 6 stages; 3 or 4 workgroups per CU with BK 32; and raised
// wave priority around the MFMAs were all slower than 128x128, BK 64,
// 2 stages, 2 independent 4-wave workgroups per CU)
using SkSmall = SkConfig<WAMC_SK_BM, WAMC_SK_BN, WAMC_SK_BK, WAMC_SK_STAGES, WAMC_SK_WGM, WAMC_SK_WGN>;
using SkBig = SkConfig<256, 256, 32, 4, 2, 4>;
using SkWide = SkConfig<256, 256, 64, 2, 2, 2>;
static_assert(SkWide::kIl && SkWide::kP == 256, "one 4-wave workgroup per CU with interleaved loads");
// The 256x256 tiles run on one 4-wave workgroup per CU (128x128 per wave,
// loads interleaved with the MFMAs) rather than 8 waves (measured at
// d = 3072, 16k rows: QKV 916 -> 874 us, out-projection 395 -> 357, MLP up
// 1289 -> 1211, MLP down 1270 -> 1114; at 2.5-2.8k rows they lose to the
// 128x128 tiles, except as the pieces of a long-K split, below).
#ifndef WAMC_GEMM_WIDE4
#define WAMC_GEMM_WIDE4 1
#endif
// Long-K projections with few 256x256 tiles: each tile cut into S K-pieces
// (S x tiles <= one workgroup per CU) that store f32 planes, reduced in piece
// order by the split-K path's second kernel, which also does the LayerNorm
// that follows where it can.  1: where the in-workgroup split-K kernel would
// not run; 2: also in its place.
#ifndef WAMC_GEMM_WIDE_PLANES
#define WAMC_GEMM_WIDE_PLANES 1
#endif
// Short-K residual projections whose plane reduction also does the LayerNorm
// that follows (the out-projection and adaLN-2) take the same split
#ifndef WAMC_WIDE_PLANES_LN
#define WAMC_WIDE_PLANES_LN 0
#endif
// QKV and MLP-up projections with at least this many 256x256 tiles (over the
// rows known to be valid) also take them; 0: only from two full rounds on
#ifndef WAMC_WIDE_MIN_TILES
#define WAMC_WIDE_MIN_TILES 0
#endif

GemmScratch gemm_scratch(int B, int rows_cap, int d, int F) {
  GemmScratch s{};
  if (rows_cap <= 0) return s;
  const int widest = max(3 * d, F);
  // arrival counters: one per output tile of the smallest tile at rows_cap rows
  s.counters = B * ((rows_cap + 127) / 128) * ((widest + 127) / 128);
  s.counter_bytes = static_cast<size_t>(s.counters) * sizeof(int);
  // partial tiles: at most two rounds of resident workgroups' worth of pieces
  // (fewer for small shapes: tiles x the most pieces per tile)
  const size_t small = std::min<size_t>(kSkSlotRounds * SkSmall::kP, static_cast<size_t>(s.counters) * kSkMaxSplit) *
                       SkSmall::kTileBytes;
  const size_t tiles_big = static_cast<size_t>(B) * ((rows_cap + 255) / 256) * ((widest + 255) / 256);
  const size_t big = kGemmBig ? std::min<size_t>(kSkSlotRounds * SkBig::kP, tiles_big * kSkMaxSplit) * SkBig::kTileBytes : 0;
  s.partial_bytes = std::max(small, big);
  return s;
}

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN>
static void launch_sk(GemmEpi epi, const GemmArgs& g, hipStream_t s) {
  using Cfg = SkConfig<BM, BN, BK, STAGES, WGM, WGN>;
  const int B = g.M / g.rows_cap;
  const long long tiles_cap = static_cast<long long>(B) * ((g.rows_cap + BM - 1) / BM) * ((g.Nout + BN - 1) / BN);
  // One workgroup per tile at the most rows, at least P so that few tiles
  // can be split, at most WAMC_SK_GRID_ROUNDS rounds of P (the workgroups
  // loop), a multiple of the 8 XCDs.  With a long K the grid also makes room
  // for the split of the tail (the split the kernel derives, given that
  // room): at 2808 rows the d=1536 down projection's 264 tiles of 140
  // k-tiles run as 792 pieces, 126.7 -> 118.9 us.  With a short K the
  // partial-tile traffic and fix-up of a split cost more than they save (the
  // QKV tail at 2458 rows: 47.1 -> 52.5 us as two-piece tiles), so the grid
  // leaves no room for one.
  constexpr long long P = Cfg::kP;
  const long long cap = static_cast<long long>(WAMC_SK_GRID_ROUNDS) * P;
  const long long ndp = tiles_cap / P * P, r = tiles_cap - ndp;
  const long long slots = std::min<long long>(static_cast<long long>(g.sk_partial_bytes / Cfg::kTileBytes), kSkSlotRounds * P);
  const long long room = std::max<long long>(std::min(cap - ndp, slots), 0);
  const int nk = g.K / BK;
  const int S = nk >= kSkLongK && r > 0 && r <= room
                    ? sk_split(static_cast<int>(r), nk, static_cast<int>(P), static_cast<int>(room))
                    : 1;
  const long long items = ndp + r * S;
  const unsigned grid = static_cast<unsigned>((std::min(std::max(items, P), cap) + 7) / 8 * 8);
  constexpr int NT = Cfg::kThreads;
  WAMC_EPI_DISPATCH(epi, (launch(gemm_bf16_sk_kernel<E, BM, BN, BK, STAGES, WGM, WGN>, grid, NT, 0, s, g)));
}

// ---------------------------------------------------------------------------
// fp32 GEMM (VALU)
// ---------------------------------------------------------------------------

constexpr int kFBM = 64, kFBN = 64, kFBK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  const int tiles_m = (g.M + kFBM - 1) / kFBM, tiles_n = (g.Nout + kFBN - 1) / kFBN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kFBM, n0 = tn * kFBN;
  if (tile_empty(g, m0, kFBM)) return;
  __shared__ float As[kFBK][kFBM + 4];
  __shared__ float Ws[kFBK][kFBN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* A = static_cast<const float*>(g.a);
  const float* W = static_cast<const float*>(g.w);
  const int K = g.K;
  float acc[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  for (int k0 = 0; k0 < K; k0 += kFBK) {
    const int gk = k0 + lk;
    float4 va = make_float4(0, 0, 0, 0), vw = make_float4(0, 0, 0, 0);
    if (m0 + lr < g.M && gk < K) va = *reinterpret_cast<const float4*>(A + static_cast<size_t>(m0 + lr) * K + gk);
    if (n0 + lr < g.Nout && gk < K) vw = *reinterpret_cast<const float4*>(W + static_cast<size_t>(n0 + lr) * K + gk);
    As[lk + 0][lr] = va.x; As[lk + 1][lr] = va.y; As[lk + 2][lr] = va.z; As[lk + 3][lr] = va.w;
    Ws[lk + 0][lr] = vw.x; Ws[lk + 1][lr] = vw.y; Ws[lk + 2][lr] = vw.z; Ws[lk + 3][lr] = vw.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; w[i] = Ws[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    const RowInfo ri = row_info(g, m);
#pragma unroll
    for (int j = 0; j < 4; ++j) epilogue<EPI, float>(g, ri, m, n0 + tx * 4 + j, acc[i][j]);
  }
}

// ---------------------------------------------------------------------------

static const char* gemm_name(const GemmArgs& g, GemmEpi e) {
  switch (e) {
    case EPI_QKV: return "gemm_qkv";
    case EPI_GELU: return "gemm_up_gelu";
    case EPI_RESID_OUT: return "gemm_out_resid";
    case EPI_RESID_DOWN: return "gemm_down_resid";
    case EPI_KV: return "gemm_text_kv";
    case EPI_STORE: return "gemm_ca_q";
    default: return "gemm_ca_out";
  }
}

template <int BM, int BN, int BK, int STAGES>
static void launch_dtl(GemmEpi epi, const GemmArgs& g, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(((g.M + BM - 1) / BM) * ((g.Nout + BN - 1) / BN));
  WAMC_EPI_DISPATCH(epi, (launch(gemm_bf16_dtl_kernel<E, BM, BN, BK, STAGES>, grid, kGemmThreads, 0, s, g)));
}

#ifndef WAMC_GEMM_TILE
#define WAMC_GEMM_TILE 0
#endif
#ifndef WAMC_GEMM_SPLITK
#define WAMC_GEMM_SPLITK 1
#endif
#ifndef WAMC_GEMM_KS2
#define WAMC_GEMM_KS2 1
#endif
constexpr bool kSplitK = WAMC_GEMM_SPLITK != 0;

// Tile shape per GEMM.  128x256 / 256x128 tiles stage a third fewer bytes per
// FLOP through LDS, but measured on the d=1536 shapes (M ~ 2.5k) every GEMM
// ran faster on 128x128 tiles, so that is the default; the others stay
// selectable for larger workloads.
static int pick_tile(const GemmArgs& g) {
  (void)g;
  return WAMC_GEMM_TILE != 0 ? WAMC_GEMM_TILE : 1;
}

// 128x192 tiles (4 waves of 64x96, two resident workgroups per CU as for
// 128x128) when, over the rows known to be valid, they need fewer rounds of
// the 512 resident workgroups by more than their 1.5x larger tiles cost: the
// QKV projection at 2458 rows is 720 tiles of 128x128 (1.4 rounds, run as
// two) or 480 of 128x192 (one round).  Only the QKV and GELU epilogues take
// them: with the residual epilogues the 64x96 wave tile spills.
static bool wide_tiles_pay(const GemmArgs& g, long long rows_known) {
  constexpr long long P = SkConfig<128, 192, 64, 2, 2, 2>::kP;
  static_assert(SkConfig<128, 192, 64, 2, 2, 2>::kP == SkConfig<128, 128, 64, 2, 2, 2>::kP, "same residency");
  const long long mt = static_cast<long long>(g.M / g.rows_cap) * ((rows_known + 127) / 128);
  const long long r128 = (mt * ((g.Nout + 127) / 128) + P - 1) / P;
  const long long r192 = (mt * ((g.Nout + 191) / 192) + P - 1) / P;
  return g.sk_partial_bytes >= SkConfig<128, 192, 64, 2, 2, 2>::kTileBytes && 3 * r192 < 2 * r128;
}

hipError_t launch_gemm(bool bf16, GemmEpi epi, const GemmArgs& g, hipStream_t s, KernelTimer* timer, bool* ln_done) {
  if (ln_done) *ln_done = false;
  if (g.M <= 0 || g.Nout <= 0) return hipSuccess;
  // Kernel choice from the tile count at rows_cap rows (measured on the d=1536
  // shapes).  With few tiles, the split-K path with a separate reduction
  // (parts_plan).  When the 128x128 tiles fit the 256 CUs in one round, the
  // in-workgroup split-K kernel gives every SIMD two waves without a trip
  // through memory; with a long K and at most half the CUs' worth of tiles the
  // work-balanced kernel, which splits K over more workgroups, is faster.
  // Otherwise the work-balanced kernel sizes its work from k_eff on the device.
  const bool dtl_ok = bf16 && g.K % 64 == 0 && !kForceGeneric;
  const long long t128 = static_cast<long long>((g.M + 127) / 128) * ((g.Nout + 127) / 128);
  const bool use_ks2 = dtl_ok && kSplitK && WAMC_GEMM_KS2 && t128 <= 256 && g.K >= 2 * 64 &&
                       (g.K < 4096 || t128 > 128);
  const PartsPlan pp = dtl_ok ? parts_plan(epi, g, use_ks2) : PartsPlan{1, 64};
  const bool use_sk = dtl_ok && WAMC_GEMM_SK && g.sk_partial && g.sk_counters &&
                      g.sk_partial_bytes >= SkSmall::kTileBytes;
  // 256-wide tiles need d >= 256 (a QKV tile crosses at most one of the Q|K|V edges).  They are
  // chosen from the rows known on the host to be valid: a launch sized for many more rows than
  // k_eff turns out to be would otherwise run 256-row tiles over a few rows (2.4x slower at 32 rows)
  const long long rows_known = g.k_eff ? std::min(g.rows_lo, g.rows_cap) : g.rows_cap;
  const long long t256 = static_cast<long long>(g.M / g.rows_cap) * ((rows_known + 255) / 256) *
                         ((g.Nout + 255) / 256);
  const bool big = kGemmBig && g.d_model >= 256 && g.sk_partial_bytes >= SkBig::kTileBytes && t256 >= 2 * SkBig::kP;
  const bool wide_few = WAMC_WIDE_MIN_TILES > 0 && g.d_model >= 256 && g.sk_partial_bytes >= SkWide::kTileBytes &&
                        t256 >= WAMC_WIDE_MIN_TILES && (epi == EPI_QKV || epi == EPI_GELU);
  const bool wide4 = (big || wide_few) && WAMC_GEMM_WIDE4;
  // pieces per 256x256 tile of a long-K projection (1: no such split)
  int wps = 1;
  const long long t256_cap = static_cast<long long>(g.M / g.rows_cap) * ((g.rows_cap + 255) / 256) *
                             ((g.Nout + 255) / 256);
  // (a long K, or a residual projection whose reduction also runs the LayerNorm that follows)
  const bool planes_pay = g.K / 64 >= kSkLongK || (WAMC_WIDE_PLANES_LN && parts_ln_fuses(epi, g));
  if (WAMC_GEMM_WIDE_PLANES && use_sk && pp.S <= 1 && !big && g.d_model >= 256 && planes_pay &&
      (!use_ks2 || WAMC_GEMM_WIDE_PLANES >= 2) && t256_cap > 0) {
    const long long plane = static_cast<long long>(g.M) * g.Nout * 4;
    long long smax = std::min<long long>((g.K / 64) / kPartsMinIters, kPartsMaxSplit);
    smax = std::min<long long>(smax, static_cast<long long>(g.sk_partial_bytes) / plane);
    // taken where the tiles at rows_cap rows split at least two ways; the
    // count itself comes from k_eff on the device (planes_split), so a launch
    // sized for every token still splits its k_eff rows' tiles as far as they
    // go (the union rule, k_eff between its larger budget and N)
    if (std::min<long long>(SkWide::kP / t256_cap, smax) >= 2) wps = static_cast<int>(smax);
  }
  TimedLaunch t(timer, gemm_name(g, epi), s, pp.S > 1 || wps > 1);   // the split-K paths launch two kernels
  // second kernel of the split-K paths: planes summed in piece order, epilogue
  // (and the LayerNorm after a residual, where it fuses)
  auto reduce_parts = [&](const GemmArgs& gp) {
    if (parts_ln_fuses(epi, g)) {
      const int nc = row_chunks(g.d_model);
      if (epi == EPI_RESID_OUT) launch_parts_resid_ln<EPI_RESID_OUT>(gp, nc, s);
      else if (epi == EPI_RESID_DOWN) launch_parts_resid_ln<EPI_RESID_DOWN>(gp, nc, s);
      else launch_parts_resid_ln<EPI_RESID_PLAIN>(gp, nc, s);
      if (ln_done) *ln_done = true;
    } else {
      const long long groups = static_cast<long long>(g.M) * (g.Nout / 4);
      const unsigned eg = static_cast<unsigned>(std::min<long long>((groups + 255) / 256, 2048));
      WAMC_EPI_DISPATCH(epi, (launch(gemm_parts_epilogue_kernel<E>, eg, 256, 0, s, gp)));
    }
  };
  if (pp.S > 1) {
    GemmArgs gp = g;
    gp.parts = pp.S;
    const long long tiles = static_cast<long long>(g.M / g.rows_cap) * ((g.rows_cap + pp.bm - 1) / pp.bm) *
                            ((g.Nout + kPartsBN - 1) / kPartsBN);
    const unsigned grid = static_cast<unsigned>(tiles * pp.S);
    if (pp.bm == 128) launch(gemm_bf16_parts_kernel<128, kPartsBN, kPartsBK, 2, 2, 2>, grid, 256, 0, s, gp);
    else launch(gemm_bf16_parts_kernel<64, kPartsBN, kPartsBK, 2, 2, 2>, grid, 256, 0, s, gp);
    reduce_parts(gp);
  } else if (wps > 1) {
    GemmArgs gp = g;
    gp.parts = -wps;   // at most wps pieces a tile, the count from k_eff
    // tiles x pieces <= max(one workgroup per CU, the tiles at rows_cap rows)
    const unsigned grid = static_cast<unsigned>((std::max<long long>(SkWide::kP, t256_cap) + 7) / 8 * 8);
    WAMC_EPI_DISPATCH(epi, (launch(gemm_bf16_sk_kernel<E, 256, 256, 64, 2, 2, 2>, grid, 256, 0, s, gp)));
    reduce_parts(gp);
  } else if (!use_ks2 && use_sk && wide4) {
    launch_sk<256, 256, 64, 2, 2, 2>(epi, g, s);
  } else if (!use_ks2 && use_sk && big) {
    launch_sk<256, 256, 32, 4, 2, 4>(epi, g, s);
  } else if (!use_ks2 && use_sk && (epi == EPI_QKV || epi == EPI_GELU) && wide_tiles_pay(g, rows_known)) {
    launch_sk<128, 192, 64, 2, 2, 2>(epi, g, s);
  } else if (!use_ks2 && use_sk) {
    launch_sk<WAMC_SK_BM, WAMC_SK_BN, WAMC_SK_BK, WAMC_SK_STAGES, WAMC_SK_WGM, WAMC_SK_WGN>(epi, g, s);
  } else if (use_ks2) {
    const unsigned grid = static_cast<unsigned>(t128);
    WAMC_EPI_DISPATCH(epi, (launch(gemm_bf16_dtl_ks2_kernel<E, 64, 2>, grid, kKs2Threads, 0, s, g)));
  } else if (dtl_ok) {
    switch (pick_tile(g)) {
      case 2: launch_dtl<128, 256, 32, 3>(epi, g, s); break;
      case 3: launch_dtl<256, 128, 32, 3>(epi, g, s); break;
      case 4: launch_dtl<128, 256, 64, 2>(epi, g, s); break;
      case 5: launch_dtl<256, 128, 64, 2>(epi, g, s); break;
      default: launch_dtl<128, 128, kDtlBK, kGemmStages>(epi, g, s); break;
    }
  } else if (bf16) {
    const unsigned grid = static_cast<unsigned>(((g.M + kBM - 1) / kBM) * ((g.Nout + kBN - 1) / kBN));
    WAMC_EPI_DISPATCH(epi, (launch(gemm_bf16_kernel<E>, grid, kGemmThreads, 0, s, g)));
  } else {
    const unsigned grid = static_cast<unsigned>(((g.M + kFBM - 1) / kFBM) * ((g.Nout + kFBN - 1) / kFBN));
    WAMC_EPI_DISPATCH(epi, (launch(gemm_f32_kernel<E>, grid, 256, 0, s, g)));
  }
  return hipGetLastError();
}

}  // namespace wamc
