// Attention of the refreshed queries over all N cached keys.
//
// WAM-Cache (paperpeel 2610.11401) §3: each query attends over all S_v keys
// and values; §4.4: a refreshed query attends over retained K/V of
// unrefreshed tokens and the fresh K/V of refreshed ones (the QKV epilogue
// has already written the fresh rows into the cache).  Non-causal, no mask.
//
// bf16 path (head_dim 128): flash-style, one workgroup of 8 waves per
// (128-query tile, head, episode); two groups of 4 waves x 32 queries take
// alternate 64-key tiles and merge (o, max, sum) at the end; online softmax
// in the log2 domain, f32.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K is the A operand (read from
//     LDS), Q^T the B operand (held in registers for the whole sweep).  The
//     result layout gives each lane one query and 32 of the tile's keys, so
//     the row max / row sum need one cross-half exchange only.
//   * O^T += V^T P^T on the same MFMA: P^T is taken straight from the S^T
//     accumulator registers (converted to bf16); the V^T A fragments are
//     read from the V tile, kept in LDS in its own [key][dh] layout, by
//     gfx950's transposing LDS read (ds_read_b64_tr_b16, two per fragment).
//   * K and V tiles go global -> LDS by direct loads, double-buffered, one
//     barrier per tile.
//   * Per tile: both halves of S first, each MFMA followed by one LDS read
//     for the next phase; one max per tile (lazy rescale); the second
//     half's exponentials between the first half's P V MFMAs.  Only the
//     ragged last tile is masked, in its own instantiation.
// fp32 path: one wavefront per query row with a VALU online softmax.
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace wamc {

constexpr float kLog2e = 1.4426950408889634f;

constexpr int kAttnThreads = 256;
constexpr int kAttnQ = 128;            // queries per workgroup
constexpr int kAttnKeys = 64;          // keys per tile
constexpr int kDh = 128;

// Lazy rescaling: the running max only moves when a tile's max exceeds it by
// more than 2^kLazy in probability (log2 units), so most tiles skip the
// rescale of the output accumulators; exp2 arguments stay <= kLazy.
constexpr float kLazy = 8.0f;
#ifndef WAMC_ATTN_GROUPS
#define WAMC_ATTN_GROUPS 2
#endif
// key-split groups of 4 waves per workgroup: 2 (one 8-wave workgroup per CU,
// the groups take alternate key tiles and merge) or 1 (two independent
// 4-wave workgroups per CU)
constexpr int kGroups = WAMC_ATTN_GROUPS;
static_assert(kGroups == 1 || kGroups == 2, "one or two key groups");
constexpr int kAttnPerCu = 2 / kGroups;         // resident workgroups per CU
constexpr int kAttnThreads2 = kAttnThreads * kGroups;
constexpr int kKsBytes = kAttnKeys * kDh * 2;   // one K or V tile, 256-byte rows, XOR-swizzled chunks

typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte chunk c (0..15) of K row r lives at chunk c ^ (r & 15): the 16 rows
// of one ds_read_b128 phase then cover all 64 banks.
__device__ __forceinline__ int ks_chunk(int row, int c) { return row * 16 + (c ^ (row & 15)); }

// 16-byte chunk c of V row r lives at chunk c ^ ((r & 3) << 2).  A
// transposing read (below) has the 32 lanes of each half-wave fetch 8 bytes
// from 4 consecutive rows x 8 chunk halves; the XOR spreads those 4 rows over
// the 4 quarters of the 256-byte bank window, so the 32 reads are disjoint.
__device__ __forceinline__ int vs_chunk(int row, int c) { return row * 16 + (c ^ ((row & 3) << 2)); }

// ds_read_b64_tr_b16, as measured on gfx950: within each group of 16 lanes,
// result lane 4*a + e receives in its slot j (j-th 16-bit element of the
// 64 bits) element e of the 4 elements read by lane 4*j + a of the group.
typedef short attn_v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) attn_v4i16_t lds_v4i16_t;

// Schedule (stream-K over the key tiles).  The active (query tile, head,
// episode) units -- only tiles holding refreshed rows count, read from k_eff
// on the device -- each have `ntiles` 64-key tiles; the T * ntiles (unit,
// key tile) steps, in unit order, are cut into G equal contiguous ranges,
// one per workgroup.  With at least P = 256 units (one round of the CUs),
// G = P, so every CU gets the same number of tile steps whatever T is; a
// range holds whole units and at most two partial ones (its first and its
// last).  With fewer units, G = T * C: every unit is cut into C equal key
// ranges, C from a cost model (rounds of the T*C pieces x (fixed piece cost
// + key tiles per piece) + merge cost per piece).  A unit covered by several
// ranges is completed by the last of its pieces to arrive, which merges the
// partial (o, max, sum) of the pieces in key order, so the result does not
// depend on arrival order.  Without scratch for partials, G = T (one unit
// per workgroup).
#ifndef WAMC_ATTN_MAX_SPLIT
#define WAMC_ATTN_MAX_SPLIT 16
#endif
#ifndef WAMC_ATTN_PIECE_COST
#define WAMC_ATTN_PIECE_COST 8
#endif
#ifndef WAMC_ATTN_MERGE_COST
#define WAMC_ATTN_MERGE_COST 2
#endif
#ifndef WAMC_ATTN_STREAMK
#define WAMC_ATTN_STREAMK 1
#endif
constexpr int kAttnP = 256 * kAttnPerCu;        // resident workgroups
constexpr int kAttnStreamUnits = 256;            // from one unit per CU on: stream-K over all P workgroups
constexpr int kAttnMinTiles = 4;                 // fewest key tiles per piece
constexpr int kAttnMaxSplit = WAMC_ATTN_MAX_SPLIT;
constexpr int kAttnPieceCost = WAMC_ATTN_PIECE_COST;   // in key tiles
constexpr int kAttnMergeCost = WAMC_ATTN_MERGE_COST;   // in key tiles, per merged piece

// First workgroup whose range [beg(v), beg(v+1)), beg(v) = v*S/G, holds
// step x: the largest v with v*S/G <= x.
__device__ __forceinline__ int attn_range_of(long long x, long long S, int G) {
  return static_cast<int>(((x + 1) * G + S - 1) / S) - 1;
}

__global__ __launch_bounds__(kAttnThreads2, kAttnPerCu) void attn_bf16_kernel(AttnArgs a, float scale2) {
  int T = 0;
  for (int bb = 0; bb < a.B; ++bb) T += (rows_of(a.k_eff, bb, a.rows_cap) + kAttnQ - 1) / kAttnQ;
  T *= a.H;
  if (T == 0) return;
  const int ntiles = (a.N + kAttnKeys - 1) / kAttnKeys;
  int G = T;
  if (a.part) {
    if (WAMC_ATTN_STREAMK && T >= kAttnStreamUnits && a.slots >= 2 * kAttnP) {
      G = kAttnP;
    } else if (T < kAttnStreamUnits) {
      // C pieces per unit within the grid and the partial slots (two per range)
      const int room = min(static_cast<int>(gridDim.x), a.slots / 2);
      const int cmax = max(1, min(min(kAttnMaxSplit, ntiles / kAttnMinTiles), room / T));
      float best = static_cast<float>(kAttnPieceCost + ntiles);
      int C = 1;
      for (int cc = 2; cc <= cmax; ++cc) {
        const float cost = static_cast<float>((T * cc + kAttnP - 1) / kAttnP) *
                               (static_cast<float>(kAttnPieceCost) + static_cast<float>(ntiles) / cc) +
                           static_cast<float>(kAttnMergeCost * cc);
        if (cost < best) {
          best = cost;
          C = cc;
        }
      }
      G = T * C;
    }
  }
  if (static_cast<int>(blockIdx.x) >= G) return;
  // consecutive ranges on one XCD: the units of one head share its K/V in that L2
  const int v = xcd_remap(blockIdx.x, G);
  const long long S_all = static_cast<long long>(T) * ntiles;
  const long long beg = v * S_all / G, end = (v + 1) * S_all / G;

  // per group and stage: a K tile, then a V tile, filled by direct-to-LDS
  // loads.  One LDS object only: with a second one the compiler cannot tell
  // the direct-to-LDS writes in flight from the reads and waits for the
  // prefetch before every tile.
  constexpr int kTileChunks = kKsBytes / 16, kStageChunks = 2 * kTileChunks;
  __shared__ uint4 kv_all[kGroups][2][kStageChunks];

  // the wave index is uniform: keep it (and what derives from it) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2, gw = wid & 3;
  const int half = lane >> 5, col = lane & 31;
  const int N = a.N, d = a.d;
  uint4* Ks0 = &kv_all[grp][0][0];
  uint4* Vs0 = Ks0 + kTileChunks;

  for (long long pos = beg; pos < end;) {
  if (pos != beg) __syncthreads();   // the previous unit's exchange area is read
  const int unit_all = static_cast<int>(pos / ntiles);
  const long long ubeg = static_cast<long long>(unit_all) * ntiles, uend = ubeg + ntiles;
  const int kt0 = static_cast<int>(pos - ubeg);
  const int kt1 = static_cast<int>(min(end, uend) - ubeg);
  const bool first_seg = pos == beg;
  pos = min(end, uend);
  int unit = unit_all;
  // unit -> (episode, head, query tile), query tile fastest: the tiles of one
  // head run on one XCD and share its K/V in that L2
  int b = 0, rt = 1;
  {
    int u = unit;
    for (b = 0; b < a.B; ++b) {
      rt = (rows_of(a.k_eff, b, a.rows_cap) + kAttnQ - 1) / kAttnQ;
      if (u < rt * a.H) break;
      u -= rt * a.H;
    }
    unit = u;   // index within the episode
  }
  const int h = unit / rt, qt = unit - h * rt;
  const int rows = rows_of(a.k_eff, b, a.rows_cap);
  const int q0 = qt * kAttnQ;
  const bf16_t* Kc = static_cast<const bf16_t*>(a.k_cache) + static_cast<size_t>(b) * N * d + h * kDh;
  const bf16_t* Vc = static_cast<const bf16_t*>(a.v_cache) + static_cast<size_t>(b) * N * d + h * kDh;

  // Q^T fragments: lane (half, col) = query q0 + gw*32 + col,
  // k-step s slot j <-> dh = s*16 + half*8 + j
  const int qrow = q0 + gw * 32 + col;
  const bf16_t* Qp = static_cast<const bf16_t*>(a.q) + (static_cast<size_t>(b) * a.rows_cap + qrow) * d + h * kDh;
  uint4 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = qrow < rows ? *reinterpret_cast<const uint4*>(Qp + s * 16 + half * 8) : make_uint4(0, 0, 0, 0);

  const int iters = (kt1 - kt0 + kGroups - 1) / kGroups;
  // group grp takes tiles kt0 + grp, kt0 + grp + 2, ... below kt1
  auto issue_k = [&](int it, int stage) {
    const int t = kt0 + it * kGroups + grp;
    if (t >= kt1) return;
    // 64 rows x 16 chunks = 1024 chunks, 4 per thread; instruction i of wave
    // gw fills LDS chunks (i*4 + gw)*64 + lane
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = (i * 4 + gw) * 64 + lane;
      const int row = c >> 4, ch = (c & 15) ^ (row & 15);
      const int key = min(t * kAttnKeys + row, N - 1);   // rows past N: a valid row, masked later
      const bf16_t* src = Kc + static_cast<size_t>(key) * d + ch * 8;
      uint4* dst = Ks0 + stage * kStageChunks + (i * 4 + gw) * 64;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)(dst), 16, 0, 0);
    }
  };
  // V tile rows in the same order, swizzled by vs_chunk
  auto issue_v = [&](int it, int stage) {
    const int t = kt0 + it * kGroups + grp;
    if (t >= kt1) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = (i * 4 + gw) * 64 + lane;
      const int row = c >> 4, ch = (c & 15) ^ ((row & 3) << 2);
      const int key = min(t * kAttnKeys + row, N - 1);   // rows past N: a valid row, its probability is 0
      const bf16_t* src = Vc + static_cast<size_t>(key) * d + ch * 8;
      uint4* dst = Vs0 + stage * kStageChunks + (i * 4 + gw) * 64;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t*)(dst), 16, 0, 0);
    }
  };
  // Transposing reads of V: lane (16*G + 4*j + a) reads 4 dh of one key row;
  // G = 2*h2 + g1 picks the half-wave h2 (the MFMA's k-half) and the 16-dh
  // half g1 of a 32-dh block, j the key within a group of 4, a the 4-dh
  // quarter.  Byte offset within a tile: row*256 + swizzled chunk*16 +
  // (a & 1)*8, with row = (keys before the group) + 4*h2 + j and chunk
  // 4*db + 2*g1 + (a >> 1); the XOR of vs_chunk only touches the chunk's
  // bits 2-3, so the chunk is 4*(db ^ j) + 2*g1 + (a >> 1).
  const int tr_g = lane >> 4, tr_j = (lane >> 2) & 3, tr_a = lane & 3;
  const int tr_base = ((tr_g >> 1) * 4 + tr_j) * 256 + (tr_g & 1) * 32 + tr_a * 8;
  int tr_db[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) tr_db[db] = tr_base + ((db ^ tr_j) << 6);

  // running max in raw logit units (the softmax scale is folded into exp2)
  float m_run = -INFINITY, l_run = 0.f;
  const float lazy = kLazy / scale2;
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_t{};

  // One 64-key tile t held in LDS stage `stage`.  Both 32-key halves are
  // multiplied first (S^T = K Q^T) and the running max moves once per tile.
  // LDS reads are issued a phase ahead of the MFMAs that consume them (the V^T
  // fragments of a half while the previous products run), and the
  // exponentials of the second half are computed while the P V products of
  // the first half run on the matrix pipe.  `ragged` is true only for the
  // last tile when N is not a multiple of 64 (a separate instantiation, so
  // full tiles carry no per-element key test).
  auto tile_step = [&](int t, int stage, auto ragged, int it) {
    const uint4* Ks = Ks0 + stage * kStageChunks;
    auto read_k = [&](int kb, bf16x8_t (&kf)[8]) {
#pragma unroll
      for (int s = 0; s < 8; ++s) kf[s] = __builtin_bit_cast(bf16x8_t, Ks[ks_chunk(kb * 32 + col, 2 * s + half)]);
    };
    // V^T fragment (tt, db) of half kb: dh row db*32 + col, slot j <-> key
    // kb*32 + 16*tt + (j/4)*8 + half*4 + j%4, the key order of the P^T
    // fragment; slots 0-3 and 4-7 are one transposing read each
    const char* Vb = reinterpret_cast<const char*>(Vs0 + stage * kStageChunks);
    auto read_v = [&](int kb, bf16x8_t (&vf)[8]) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const char* p0 = Vb + tr_db[db] + (kb * 32 + 16 * tt) * 256;
          const attn_v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p0));
          const attn_v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p0 + 8 * 256));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          vf[tt * 4 + db] = __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
        }
    };
    auto qk = [&](const bf16x8_t (&kf)[8]) {
      f32x16_t acc = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], __builtin_bit_cast(bf16x8_t, qf[s]), acc, 0, 0, 0);
      return acc;
    };
    bf16x8_t ka[8], kb1[8], v0[8], v1[8];
    read_k(0, ka);
    __builtin_amdgcn_sched_barrier(0);
    // S for the first half, each MFMA followed by one K read of the second
    // half; then S for the second half, each MFMA followed by one V^T read of
    // the first half (each read lands in registers its MFMA has just freed)
    read_k(1, kb1);
    f32x16_t s0 = qk(ka);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_v(0, v0);
    f32x16_t s1 = qk(kb1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    // s<kb>[v]: key t*64 + kb*32 + (v/4)*8 + half*4 + v%4, query col
    if constexpr (decltype(ragged)::value) {
      const int kbase = t * kAttnKeys;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kv = kbase + (v / 4) * 8 + half * 4 + (v % 4);
        if (kv >= N) s0[v] = -INFINITY;
        if (kv + 32 >= N) s1[v] = -INFINITY;
      }
    }
    float tmax = s0[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, s0[v]);
#pragma unroll
    for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s1[v]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    if (__ballot(tmax > m_run + lazy)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale2);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    const float mb = -m_run * scale2;
    // P^T fragment tt of half kb covers keys kb*32 + 16*tt + (j/4)*8 + half*4 + j%4
    auto probs = [&](f32x16_t& sacc, bf16x8_t (&pk)[2]) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[v], scale2, mb));
        sacc[v] = p;
        l_run += p;
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint4 w;
        w.x = pack_bf16x2(sacc[8 * tt + 0], sacc[8 * tt + 1]);
        w.y = pack_bf16x2(sacc[8 * tt + 2], sacc[8 * tt + 3]);
        w.z = pack_bf16x2(sacc[8 * tt + 4], sacc[8 * tt + 5]);
        w.w = pack_bf16x2(sacc[8 * tt + 6], sacc[8 * tt + 7]);
        pk[tt] = __builtin_bit_cast(bf16x8_t, w);
      }
    };
    auto pv = [&](const bf16x8_t (&vf)[8], const bf16x8_t (&pk)[2]) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[tt * 4 + db], pk[tt], o[db], 0, 0, 0);
    };
    bf16x8_t p0[2], p1[2];
    probs(s0, p0);
    read_v(1, v1);
    // The next tile's loads go out here, after this tile's last LDS read:
    // the compiler cannot match the transposing reads against direct-to-LDS
    // writes in flight and would wait for every such write before them.
    issue_k(it + 1, (it + 1) & 1);
    issue_v(it + 1, (it + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    pv(v0, p0);
    probs(s1, p1);
    // one MFMA of the first half's P V, then a share of the second half's
    // exponentials, eight times
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 3);
    }
    __builtin_amdgcn_sched_barrier(0);
    pv(v1, p1);
  };

  issue_k(0, 0);
  issue_v(0, 0);
  // The ragged tile, when there is one in this piece, is tile ntiles - 1 and
  // falls in the last iteration; that iteration runs after the loop, both
  // groups in the masking instantiation, so that each path through the loop
  // body issues its prefetch after its own last LDS read (two instantiations
  // in one body would be laid out one after the other under an exec mask,
  // and the second would wait for the first's prefetch).
  const int full_iters = (kt1 == ntiles && ntiles * kAttnKeys > N) ? iters - 1 : iters;
  for (int it = 0; it < full_iters; ++it) {
    // this thread's K and V loads of tile `it` have landed in LDS ...
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));   // vmcnt(0)
    // ... and everybody's, and every wave is done with the stage that the
    // prefetch of tile it + 1 (issued inside the step) overwrites
    __builtin_amdgcn_s_barrier();
    const int t = kt0 + it * kGroups + grp;
    if (t < kt1) tile_step(t, it & 1, std::false_type{}, it);
  }
  if (full_iters < iters) {
    const int it = full_iters;
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));   // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    const int t = kt0 + it * kGroups + grp;
    if (t < kt1) tile_step(t, it & 1, std::true_type{}, it);
  }

  // merge the two key groups: group 1 hands (o, m, l) to group 0 through LDS
  // (o in the first 64 KiB of the tile buffers, 64 floats per lane; m and l
  // after it)
  __syncthreads();
  float* xo = reinterpret_cast<float*>(&kv_all[0][0][0]);
  float* xml = xo + 4 * 64 * 64;
  float m = 0.f, e0 = 0.f, e1 = 0.f, l = 0.f;
  if constexpr (kGroups == 2) {
    static_assert(kGroups != 2 || 4 * 64 * 64 * 4 + 4 * 2 * 64 * 4 + 16 <= sizeof(kv_all),
                  "exchange of o, m, l and the flag fits the tile buffers");
    if (grp == 1) {
      float* dst = xo + static_cast<size_t>(gw) * 64 * 64 + lane;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[(db * 16 + v) * 64] = o[db][v];
      xml[(gw * 2 + 0) * 64 + lane] = m_run;
      xml[(gw * 2 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (grp == 0) {
      const float m1 = xml[(gw * 2 + 0) * 64 + lane], l1 = xml[(gw * 2 + 1) * 64 + lane];
      m = fmaxf(m_run, m1);
      e0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m) * scale2);
      e1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - m) * scale2);
      const float lsum = l_run * e0 + l1 * e1;
      l = lsum + __shfl_xor(lsum, 32, kWave);
    }
  } else {
    m = m_run;
    e0 = 1.f;
    l = l_run + __shfl_xor(l_run, 32, kWave);
  }
  // group 1's contribution to element (db, v) of this lane (none with one group)
  const float* src = xo + static_cast<size_t>(gw) * 64 * 64 + lane;
  auto other = [&](int db, int vv) { return kGroups == 2 ? src[(db * 16 + vv) * 64] * e1 : 0.f; };
  bf16_t* Op = static_cast<bf16_t*>(a.o) + (static_cast<size_t>(b) * a.rows_cap + qrow) * d + h * kDh;
  if (kt0 == 0 && kt1 == ntiles) {
    // the whole unit in this range: normalise and store
    if (grp == 0 && qrow < rows) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          // elements v = g4*4 .. g4*4+3: dh rows db*32 + g4*8 + half*4 + 0..3
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int vv = g4 * 4 + e;
            r[e] = (o[db][vv] * e0 + other(db, vv)) * inv;
          }
          uint2 w;
          w.x = pack_bf16x2(r[0], r[1]);
          w.y = pack_bf16x2(r[2], r[3]);
          *reinterpret_cast<uint2*>(Op + db * 32 + g4 * 8 + half * 4) = w;
        }
    }
    continue;
  }

  // part of the unit: group 0 writes this piece's (o relative to m, m, l) to
  // the range's slot (2v for its first piece, 2v + 1 for its last) as relaxed
  // system-scope atomics (coherent between the XCDs' caches without
  // cache-wide maintenance), then the arrival is counted
  const int gl = gw * 64 + lane;   // lane of group 0 holding the same queries
  float* slot_base = a.part;
  if (grp == 0) {
    float* dst = slot_base + static_cast<size_t>(2 * v + (first_seg ? 0 : 1)) * kAttnPartFloats;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const int vv = g4 * 4 + e;
          const float x0 = o[db][vv] * e0 + other(db, vv);
          const float x1 = o[db][vv + 1] * e0 + other(db, vv + 1);
          const unsigned long long w = (static_cast<unsigned long long>(__float_as_uint(x1)) << 32) | __float_as_uint(x0);
          __hip_atomic_store(reinterpret_cast<unsigned long long*>(dst) + ((db * 4 + g4) * 2 + e / 2) * 256 + gl, w,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    __hip_atomic_store(dst + 128 * 128 + gl, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(dst + 128 * 128 + 256 + gl, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  __builtin_amdgcn_s_waitcnt(0);   // the stores have reached the coherence point
  __syncthreads();
  // the ranges holding this unit: v_first .. v_last, in key order
  const int v_first = attn_range_of(ubeg, S_all, G);
  const int v_last = attn_range_of(uend - 1, S_all, G);
  const int npieces = v_last - v_first + 1;
  // past the exchanged m, l (with one group the tile buffers are free)
  int* flag = kGroups == 2 ? reinterpret_cast<int*>(xml) + 1024 : reinterpret_cast<int*>(xo);
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&a.counters[unit_all], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const int last = old == npieces - 1 ? 1 : 0;
    if (last) __hip_atomic_store(&a.counters[unit_all], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    *flag = last;
  }
  __syncthreads();
  if (!*flag || qrow >= rows) continue;
  // last piece: merge the partials in key order; with two groups group g
  // finishes dh blocks 2g, 2g+1, with one group the group does all four, two
  // blocks at a time.
  // A range that starts inside the unit holds it as its first piece (slot
  // 2v), one that starts before it as its last (slot 2v + 1).
  float mt = -INFINITY;
  for (int vc = v_first; vc <= v_last; ++vc) {
    const long long bc = vc * S_all / G;
    const float* pp = slot_base + static_cast<size_t>(2 * vc + (bc >= ubeg ? 0 : 1)) * kAttnPartFloats;
    mt = fmaxf(mt, __hip_atomic_load(pp + 128 * 128 + gl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM));
  }
  for (int blk0 = 2 * grp; blk0 < 4; blk0 += 2 * kGroups) {
  float acc[2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) acc[i][vv] = 0.f;
  float lt = 0.f;
  for (int vc = v_first; vc <= v_last; ++vc) {
    const long long bc = vc * S_all / G;
    const float* pp = slot_base + static_cast<size_t>(2 * vc + (bc >= ubeg ? 0 : 1)) * kAttnPartFloats;
    const float mc = __hip_atomic_load(pp + 128 * 128 + gl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const float lc = __hip_atomic_load(pp + 128 * 128 + 256 + gl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const float sc = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mc - mt) * scale2);
    lt += lc * sc;
    unsigned long long w[16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[i * 8 + q] = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(pp) +
                                             (((blk0 + i) * 4 + q / 2) * 2 + q % 2) * 256 + gl,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        acc[i][2 * q] += __uint_as_float(static_cast<unsigned>(w[i * 8 + q])) * sc;
        acc[i][2 * q + 1] += __uint_as_float(static_cast<unsigned>(w[i * 8 + q] >> 32)) * sc;
      }
  }
  const float inv = 1.0f / lt;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      uint2 w;
      w.x = pack_bf16x2(acc[i][g4 * 4 + 0] * inv, acc[i][g4 * 4 + 1] * inv);
      w.y = pack_bf16x2(acc[i][g4 * 4 + 2] * inv, acc[i][g4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(Op + (blk0 + i) * 32 + g4 * 8 + half * 4) = w;
    }
  }   // dh block pairs
  }   // ranges of this workgroup
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
    // with partial scratch: one round of workgroups (the kernel derives its
    // ranges from k_eff and exits the ones it does not need); without: one
    // workgroup per unit at rows_cap rows
    const long long units = static_cast<long long>((a.rows_cap + kAttnQ - 1) / kAttnQ) * a.H * a.B;
    const long long with_part = WAMC_ATTN_STREAMK ? kAttnP : std::max<long long>(units, kAttnP);
    const unsigned grid = static_cast<unsigned>(a.part ? with_part : units);
    launch(attn_bf16_kernel, grid, kAttnThreads2, 0, s, a, scale2);
  } else {
    const dim3 grid((a.rows_cap + 3) / 4, a.H, a.B);
    launch(attn_f32_kernel, grid, 256, 0, s, a, scale2);
  }
  return hipGetLastError();
}

}  // namespace wamc

namespace wamc {

AttnScratch attn_scratch(int B, int rows_cap, int H) {
  AttnScratch s{};
  if (rows_cap <= 0) return s;
  s.slots = kAttnSlotsMax;
  s.counters = B * ((rows_cap + kAttnQ - 1) / kAttnQ) * H;
  s.part_bytes = static_cast<size_t>(s.slots) * kAttnPartFloats * sizeof(float);
  s.counter_bytes = static_cast<size_t>(s.counters) * sizeof(int);
  return s;
}

}  // namespace wamc
