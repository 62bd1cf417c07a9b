// Refresh-set selection with the age bound, and age bookkeeping.
//
// WAM-Cache (paperpeel 2610.11401) §1 and §4.4: tokens whose age counter
// reached the bound G are forced into the refresh set; the set is filled by
// score.  RealtimeWAM App. D.3 "Recursive reuse": an age cap of G permits at
// most G consecutive reuses, so age is reset on refresh and incremented on
// reuse.
//
// Design (one workgroup of 1024 threads per episode):
//  * every token gets a unique 64-bit key  forced(1) | orderable score(32) |
//    (2^31-1 - index)(31), so "largest key" = forced first, then higher
//    score, then lower index; keys live in registers (up to 8 per thread, N <= 8192; larger N
//    recomputes them from global memory in each pass);
//  * the k_eff-th largest key is found by an MSB-first radix select over
//    the group it lies in (forced or not): 8-bit digit histograms in LDS
//    from the highest bit in which the group's keys differ, the bucket found
//    by a wave-wide suffix scan -- no sort at all;
//  * the refresh set = keys >= that threshold, compacted in ascending token
//    order with a block-wide ballot/popcount scan, which also yields the
//    new ages.
// Everything is integer work, so the result is bit-exact by construction.
#include "common.h"
#include "launch.h"

namespace wamc {

__device__ __forceinline__ uint64_t rank_key(float s, bool forced, int i) {
  uint32_t f = __float_as_uint(s);
  uint32_t ord;
  if ((f & 0x7fffffffu) > 0x7f800000u) {
    ord = 0u;                       // NaN: below every number
  } else {
    if (f == 0x80000000u) f = 0u;   // -0.0 ranks equal to +0.0
    ord = (f & 0x80000000u) ? ~f : (f | 0x80000000u);
  }
  return (static_cast<uint64_t>(forced) << 63) | (static_cast<uint64_t>(ord) << 31) |
         static_cast<uint64_t>(0x7fffffffu - static_cast<uint32_t>(i));
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

struct SelShared {
  uint32_t hist[3][256];     // a pass's histogram rotates through three buffers
  int red[kSelWaves];
  int red2[2][kSelWaves];    // per-wave counts of the compaction, alternating
  uint64_t red64[kSelWaves];
  uint64_t red64b[kSelWaves];
  float red4[4];
};

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
    const uint64_t w = (static_cast<uint64_t>(hi) << 32) | lo;
    v = w < v ? w : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
    const uint64_t w = (static_cast<uint64_t>(hi) << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// The count-th largest key (1 <= count < N) by an MSB-first radix select:
// passes of an 8-bit digit histogram in LDS over the keys of the group the
// answer lies in (the n_top keys with the top bit set, or the others), from
// the highest bit in which the group's keys differ; the bucket is found by a
// wave-wide suffix scan.  Once the bucket that holds the answer is taken
// whole (its size equals the rank still wanted inside it -- with distinct
// scores this happens after two or three passes), the answer is that
// bucket's smallest key, found by one block-wide minimum instead of the
// remaining passes.  key_of(j, i) gives the key of token i, held in
// register slot j when KPT > 0 (i = tid + j*1024); with KPT == 0 it is
// recomputed for every i.  All threads of the block call it.
template <int KPT, class KeyOf>
__device__ uint64_t radix_threshold(KeyOf key_of, int N, uint32_t count, uint32_t n_top, SelShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  // The answer lies among the n_top keys with the top bit set (the forced
  // tokens) when count <= n_top, else among the others at rank count - n_top.
  // The group's smallest and largest keys share every bit above the highest
  // bit in which they differ, so the first pass starts there instead of at
  // bit 63 (where the forced bit and the shared exponent bits of the scores
  // would take passes that split nothing).
  const bool top = count <= n_top;
  uint32_t remaining = top ? count : count - n_top;
  uint64_t mx = 0, mn = ~0ull;
  auto fold = [&](uint64_t key) {
    if ((key >> 63) == (top ? 1ull : 0ull)) {
      mx = key > mx ? key : mx;
      mn = key < mn ? key : mn;
    }
  };
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + j * kSelThreads;
      if (i < N) fold(key_of(j, i));
    }
  } else {
    for (int i = tid; i < N; i += kSelThreads) fold(key_of(0, i));
  }
  mx = wave_max_u64(mx);
  mn = wave_min_u64(mn);
  if (lane == 0) {
    sh.red64[wid] = mn;
    sh.red64b[wid] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    mn = sh.red64[w] < mn ? sh.red64[w] : mn;
    mx = sh.red64b[w] > mx ? sh.red64b[w] : mx;
  }
  // the first pass's histogram; every wave is past any earlier reader of it
  if (tid < 256) sh.hist[0][tid] = 0;
  __syncthreads();   // sh is reused below
  if (mx == mn) return mx;   // a group of one key
  // bits >= fixed are known: those of the group's common prefix, then each
  // pass's digit; a pass takes the (up to 8) next bits below them
  int fixed = 64 - __clzll(static_cast<long long>(mx ^ mn));   // the highest differing bit + 1 (<= 63)
  uint64_t prefix = mx & (~0ull << fixed);
  // One barrier per pass: pass p counts into buffer p%3 (zeroed during the
  // pass before) and zeroes buffer (p+1)%3, whose last readers finished
  // before the previous barrier; every wave then finds the bucket itself.
  for (int pass = 0; fixed > 0; ++pass) {
    const int shift = fixed > 8 ? fixed - 8 : 0;
    const uint64_t hi_mask = ~0ull << fixed;
    const uint32_t dmask = (1u << (fixed - shift)) - 1u;
    uint32_t* hist = sh.hist[pass % 3];
    if (tid < 256) sh.hist[(pass + 1) % 3][tid] = 0;
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int i = tid + j * kSelThreads;
        if (i < N) {
          const uint64_t key = key_of(j, i);
          if ((key & hi_mask) == prefix) atomicAdd(&hist[static_cast<uint32_t>(key >> shift) & dmask], 1u);
        }
      }
    } else {
      for (int i = tid; i < N; i += kSelThreads) {
        const uint64_t key = key_of(0, i);
        if ((key & hi_mask) == prefix) atomicAdd(&hist[static_cast<uint32_t>(key >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    // lane l owns bins 4l..4l+3; suffix sums find the bucket that holds the
    // remaining-th largest key (exactly one lane does)
    const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
    const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
    const uint32_t s4 = h0 + h1 + h2 + h3;
    uint32_t suf = s4;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t v = __shfl_down(suf, o, kWave);
      if (lane + o < kWave) suf += v;
    }
    const uint32_t above = suf - s4;
    const bool found = above < remaining && remaining <= suf;
    uint32_t sel = 0, rem = 0, whole = 0;
    if (found) {
      uint32_t c = above;
      if (c + h3 >= remaining) {
        sel = 4 * lane + 3;
      } else {
        c += h3;
        if (c + h2 >= remaining) {
          sel = 4 * lane + 2;
        } else {
          c += h2;
          if (c + h1 >= remaining) {
            sel = 4 * lane + 1;
          } else {
            c += h1;
            sel = 4 * lane;
          }
        }
      }
      const uint32_t hs = sel == 4 * lane + 3 ? h3 : sel == 4 * lane + 2 ? h2 : sel == 4 * lane + 1 ? h1 : h0;
      rem = remaining - c;
      whole = hs == rem ? 1u : 0u;
    }
    const int fl = __builtin_ctzll(__ballot(found));
    sel = __shfl(sel, fl, kWave);
    rem = __shfl(rem, fl, kWave);
    whole = __shfl(whole, fl, kWave);
    prefix |= static_cast<uint64_t>(sel) << shift;
    remaining = rem;
    fixed = shift;
    if (whole && shift > 0) {
      // every key of the bucket is selected: the answer is its minimum
      const uint64_t mask = ~0ull << shift;
      uint64_t m = ~0ull;
      if constexpr (KPT > 0) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const int i = tid + j * kSelThreads;
          if (i < N) {
            const uint64_t key = key_of(j, i);
            if ((key & mask) == prefix && key < m) m = key;
          }
        }
      } else {
        for (int i = tid; i < N; i += kSelThreads) {
          const uint64_t key = key_of(0, i);
          if ((key & mask) == prefix && key < m) m = key;
        }
      }
      m = wave_min_u64(m);
      if (lane == 0) sh.red64[wid] = m;
      __syncthreads();
      uint64_t r = ~0ull;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) r = sh.red64[w] < r ? sh.red64[w] : r;
      __syncthreads();   // sh is reused by the caller
      return r;
    }
  }
  return prefix;
}

// Ascending-order compaction of the tokens with flag_of(j, i) set into idx,
// ages reset on the set and +1 elsewhere; returns the set size.  One
// 1024-token tile at a time with a block-wide ballot/popcount scan.
template <int KPT, class FlagOf, class AgeOf>
__device__ int compact_set(FlagOf flag_of, AgeOf age_of, int N, int32_t* __restrict__ idx,
                           int32_t* __restrict__ age, SelShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  int base = 0, parity = 0;
  // one barrier per tile: the per-wave counts alternate between two arrays,
  // and a wave can only write tile t+1's counts after every wave passed the
  // barrier of tile t, that is after reading tile t-1's
  auto tile = [&](int j, int i, bool flag) {
    const uint64_t ball = __ballot(flag);
    const int wpre = __popcll(ball & ((1ull << lane) - 1ull));
    int* red = sh.red2[parity];
    parity ^= 1;
    if (lane == 0) red[wid] = __popcll(ball);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const int c = red[w];
      off += w < wid ? c : 0;
      tot += c;
    }
    if (flag) idx[base + off + wpre] = i;
    if (i < N) age[i] = flag ? 0 : age_of(j, i) + 1;
    base += tot;
  };
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (j * kSelThreads >= N) break;
      const int i = tid + j * kSelThreads;
      tile(j, i, i < N && flag_of(j, i));
    }
  } else {
    for (int t0 = 0; t0 < N; t0 += kSelThreads) {
      const int i = t0 + tid;
      tile(0, i, i < N && flag_of(0, i));
    }
  }
  for (int i = base + tid; i < N; i += kSelThreads) idx[i] = -1;
  return base;
}

// block-wide count of forced tokens (age >= G); the ages come from the
// registers ag (token tid + j*1024 in slot j) when KPT > 0
template <int KPT>
__device__ int count_forced(const int32_t* __restrict__ age, const int (&ag)[KPT > 0 ? KPT : 1], int N, int G,
                            SelShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  int nf = 0;
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) nf += (tid + j * kSelThreads < N && ag[j] >= G) ? 1 : 0;
  } else {
    for (int i = tid; i < N; i += kSelThreads) nf += age[i] >= G;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nf += __shfl_xor(nf, o, kWave);
  if (lane == 0) sh.red[wid] = nf;
  __syncthreads();
  int n = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) n += sh.red[w];
  __syncthreads();
  return n;
}

// KPT = keys held per thread in registers (N <= KPT * 1024); 0 = recompute
// the keys from global memory in every pass (any N).
// SCORED: the scores are formed here from P, U and the U partials (the last
// scoring step fused in) and written to si.score_out; otherwise read.
template <int KPT, bool SCORED>
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const float* __restrict__ score, ScoreInputs si, int32_t* __restrict__ age, int N, int k, int G,
    int rows_cap, int32_t* __restrict__ idx, int32_t* __restrict__ k_eff_out,
    int32_t* __restrict__ n_forced_out) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t eoff = static_cast<size_t>(b) * N;
  age += eoff;
  idx += eoff;
  __shared__ SelShared sh;

  constexpr int NK = KPT > 0 ? KPT : 1;
  uint64_t keys[NK];
  int ag[NK];
  float total = 0.f;
  if constexpr (KPT > 0) {
    // every token load is issued before the first use
    float pa[KPT], pb[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + j * kSelThreads;
      const size_t ic = eoff + (i < N ? i : 0);
      if constexpr (SCORED) {
        pa[j] = si.mass[ic];
        pb[j] = si.surprise[ic];
      } else {
        pa[j] = score[ic];
        pb[j] = 0.f;
      }
      ag[j] = age[i < N ? i : 0];
    }
    if constexpr (SCORED) total = usum_total(si.usum + static_cast<size_t>(b) * si.nblocks, si.nblocks, sh.red4);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + j * kSelThreads;
      keys[j] = 0;
      if (i < N) {
        float sc = pa[j];
        if constexpr (SCORED) {
          sc = combine_score(pa[j], pb[j], total, si.w_attn_norm, si.w_surprise);
          si.score_out[eoff + i] = sc;
        }
        keys[j] = rank_key(sc, ag[j] >= G, i);
      }
    }
  } else {
    if constexpr (SCORED) {
      total = usum_total(si.usum + static_cast<size_t>(b) * si.nblocks, si.nblocks, sh.red4);
      for (int i = tid; i < N; i += kSelThreads)
        si.score_out[eoff + i] = combine_score(si.mass[eoff + i], si.surprise[eoff + i], total, si.w_attn_norm,
                                               si.w_surprise);
    }
  }
  auto get_score = [&](int i) -> float {
    if constexpr (SCORED)
      return combine_score(si.mass[eoff + i], si.surprise[eoff + i], total, si.w_attn_norm, si.w_surprise);
    else
      return score[eoff + i];
  };
  const int n_forced = count_forced<KPT>(age, ag, N, G, sh);

  int ke = k > n_forced ? k : n_forced;
  if (ke > rows_cap) ke = rows_cap;
  const bool take_all = ke >= N, take_none = ke <= 0;
  auto key_of = [&](int j, int i) -> uint64_t {
    if constexpr (KPT > 0) return keys[j];
    else return rank_key(get_score(i), age[i] >= G, i);
  };
  uint64_t thr = 0;
  if (!take_all && !take_none)
    thr = radix_threshold<KPT>(key_of, N, static_cast<uint32_t>(ke), static_cast<uint32_t>(n_forced), sh);
  auto age_of = [&](int j, int i) -> int {
    if constexpr (KPT > 0) return ag[j];
    else return age[i];
  };
  compact_set<KPT>([&](int j, int i) { return take_all || (!take_none && key_of(j, i) >= thr); }, age_of, N, idx,
                   age, sh);
  if (tid == 0) {
    k_eff_out[b] = ke;
    if (n_forced_out) n_forced_out[b] = n_forced;
  }
}

// The union rule (WAM-Cache §1, §4.3, §4.4): the n_attn tokens of largest
// attention mass, the n_surprise tokens of largest surprise and the forced
// tokens, each once; k_eff = the size of the union (at most N).  Two radix
// selects on the keys  mass(32) | ~index(31)  and  surprise(32) | ~index(31)
// (same order conventions as above), then one compaction of the union.
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_union_kernel(
    const float* __restrict__ mass, const float* __restrict__ surprise, int32_t* __restrict__ age, int N,
    int n_attn, int n_surprise, int G, int32_t* __restrict__ idx, int32_t* __restrict__ k_eff_out,
    int32_t* __restrict__ n_forced_out) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t eoff = static_cast<size_t>(b) * N;
  age += eoff;
  idx += eoff;
  mass += eoff;
  surprise += eoff;
  __shared__ SelShared sh;

  constexpr int NK = KPT > 0 ? KPT : 1;
  uint64_t kp[NK], ku[NK];
  int ag[NK];
  if constexpr (KPT > 0) {
    // every token load is issued before the first use
    float pm[KPT], pu[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + j * kSelThreads, ic = i < N ? i : 0;
      pm[j] = mass[ic];
      pu[j] = surprise[ic];
      ag[j] = age[ic];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + j * kSelThreads;
      kp[j] = i < N ? rank_key(pm[j], false, i) : 0;
      ku[j] = i < N ? rank_key(pu[j], false, i) : 0;
    }
  }
  const int n_forced = count_forced<KPT>(age, ag, N, G, sh);
  auto age_of = [&](int j, int i) -> int {
    if constexpr (KPT > 0) return ag[j];
    else return age[i];
  };
  auto kp_of = [&](int j, int i) -> uint64_t {
    if constexpr (KPT > 0) return kp[j];
    else return rank_key(mass[i], false, i);
  };
  auto ku_of = [&](int j, int i) -> uint64_t {
    if constexpr (KPT > 0) return ku[j];
    else return rank_key(surprise[i], false, i);
  };
  // thresholds: ~0 selects nothing (keys never reach it), 0 selects everything
  const uint64_t kNone = ~0ull;
  uint64_t tp = kNone, tu = kNone;
  if (n_attn >= N) tp = 0;
  else if (n_attn > 0) tp = radix_threshold<KPT>(kp_of, N, static_cast<uint32_t>(n_attn), 0u, sh);
  if (n_surprise >= N) tu = 0;
  else if (n_surprise > 0) tu = radix_threshold<KPT>(ku_of, N, static_cast<uint32_t>(n_surprise), 0u, sh);
  const int ke = compact_set<KPT>(
      [&](int j, int i) {
        return age_of(j, i) >= G || (tp != kNone && kp_of(j, i) >= tp) || (tu != kNone && ku_of(j, i) >= tu);
      },
      age_of, N, idx, age, sh);
  if (tid == 0) {
    k_eff_out[b] = ke;
    if (n_forced_out) n_forced_out[b] = n_forced;
  }
}

template <bool SCORED>
static void launch_select_impl(const float* score, const ScoreInputs& si, int32_t* age, int B, int N, int k, int G,
                               int rows_cap, int32_t* idx, int32_t* k_eff, int32_t* n_forced, hipStream_t s) {
  const dim3 grid(B), block(kSelThreads);
  if (N <= 1024)
    launch(select_topk_kernel<1, SCORED>, grid, block, 0, s, score, si, age, N, k, G, rows_cap, idx, k_eff, n_forced);
  else if (N <= 2048)
    launch(select_topk_kernel<2, SCORED>, grid, block, 0, s, score, si, age, N, k, G, rows_cap, idx, k_eff, n_forced);
  else if (N <= 4096)
    launch(select_topk_kernel<4, SCORED>, grid, block, 0, s, score, si, age, N, k, G, rows_cap, idx, k_eff, n_forced);
  else if (N <= 8192)
    launch(select_topk_kernel<8, SCORED>, grid, block, 0, s, score, si, age, N, k, G, rows_cap, idx, k_eff, n_forced);
  else
    launch(select_topk_kernel<0, SCORED>, grid, block, 0, s, score, si, age, N, k, G, rows_cap, idx, k_eff, n_forced);
}

hipError_t launch_select(const float* score, int32_t* age, int B, int N, int k, int G, int rows_cap,
                         int32_t* idx, int32_t* k_eff, int32_t* n_forced, hipStream_t s) {
  launch_select_impl<false>(score, ScoreInputs{}, age, B, N, k, G, rows_cap, idx, k_eff, n_forced, s);
  return hipGetLastError();
}

hipError_t launch_select_scored(const ScoreInputs& si, int32_t* age, int B, int N, int k, int G, int rows_cap,
                                int32_t* idx, int32_t* k_eff, int32_t* n_forced, hipStream_t s) {
  launch_select_impl<true>(nullptr, si, age, B, N, k, G, rows_cap, idx, k_eff, n_forced, s);
  return hipGetLastError();
}

hipError_t launch_select_union(const float* mass, const float* surprise, int32_t* age, int B, int N, int n_attn,
                               int n_surprise, int G, int32_t* idx, int32_t* k_eff, int32_t* n_forced,
                               hipStream_t s) {
  const dim3 grid(B), block(kSelThreads);
  if (N <= 1024)
    launch(select_union_kernel<1>, grid, block, 0, s, mass, surprise, age, N, n_attn, n_surprise, G, idx, k_eff, n_forced);
  else if (N <= 2048)
    launch(select_union_kernel<2>, grid, block, 0, s, mass, surprise, age, N, n_attn, n_surprise, G, idx, k_eff, n_forced);
  else if (N <= 4096)
    launch(select_union_kernel<4>, grid, block, 0, s, mass, surprise, age, N, n_attn, n_surprise, G, idx, k_eff, n_forced);
  else if (N <= 8192)
    launch(select_union_kernel<8>, grid, block, 0, s, mass, surprise, age, N, n_attn, n_surprise, G, idx, k_eff, n_forced);
  else
    launch(select_union_kernel<0>, grid, block, 0, s, mass, surprise, age, N, n_attn, n_surprise, G, idx, k_eff, n_forced);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Ages from a caller-given refresh set (idx_override): copy the set into the
// output buffers, then age + 1 everywhere and 0 on the set.
// ---------------------------------------------------------------------------

__global__ void copy_set_kernel(const int32_t* __restrict__ idx_in, const int32_t* __restrict__ k_in,
                                int B, int N, int rows_cap, int32_t* __restrict__ idx_out,
                                int32_t* __restrict__ k_out) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < static_cast<size_t>(B) * N) idx_out[i] = idx_in[i];
  if (i < static_cast<size_t>(B)) k_out[i] = rows_of(k_in, static_cast<int>(i), rows_cap);
}

__global__ void age_increment_kernel(int32_t* __restrict__ age, size_t total) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < total) age[i] += 1;
}

__global__ void age_reset_kernel(int32_t* __restrict__ age, const int32_t* __restrict__ idx,
                                 const int32_t* __restrict__ k_eff, int N, int rows_cap) {
  const int b = blockIdx.y;
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows_of(k_eff, b, rows_cap)) return;
  const int t = idx[static_cast<size_t>(b) * N + r];
  if (t >= 0 && t < N) age[static_cast<size_t>(b) * N + t] = 0;
}

hipError_t launch_ages_from_set(const int32_t* idx_in, const int32_t* k_in, int B, int N, int rows_cap,
                                int32_t* idx_out, int32_t* k_out, int32_t* age, hipStream_t s) {
  const size_t total = static_cast<size_t>(B) * N;
  const int t = 256;
  const unsigned g = static_cast<unsigned>((total + t - 1) / t);
  if (idx_in != idx_out || k_in != k_out)
    launch(copy_set_kernel, g, t, 0, s, idx_in, k_in, B, N, rows_cap, idx_out, k_out);
  launch(age_increment_kernel, g, t, 0, s, age, total);
  launch(age_reset_kernel, dim3((rows_cap + t - 1) / t, B), t, 0, s, age, idx_out, k_out, N, rows_cap);
  return hipGetLastError();
}

}  // namespace wamc
