// Host-side launchers of the libwamc kernels and the optional kernel timer.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace wamc {

// Optional per-kernel timer, implemented in api.cpp.  While timing is on, a
// TimedLaunch scope takes a pair of HIP events from it.  The one kernel that
// the scope launches through wamc::launch carries them: hipExtLaunchKernelGGL
// stamps them with that kernel's own start and end on the device, which is
// the interval a kernel trace reports.  A scope that launches several kernels
// (`markers`) records the events around them on the stream instead.
class KernelTimer {
 public:
  virtual ~KernelTimer() = default;
  // Returns false (no events) when no event could be had.
  virtual bool begin(const char* kind, hipStream_t s, bool markers, hipEvent_t* start, hipEvent_t* stop) = 0;
  // `launched` = kernels that took the events (1 is a valid record).
  virtual void end(hipStream_t s, bool markers, hipEvent_t start, hipEvent_t stop, int launched) = 0;
};

struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  int launched = 0;
};

// The events of the TimedLaunch scope open on this host thread (null outside one).
inline thread_local LaunchEvents* t_launch_events = nullptr;

struct TimedLaunch {
  KernelTimer* t;
  hipStream_t s;
  bool markers;
  bool on = false;
  LaunchEvents ev;
  LaunchEvents* outer;
  TimedLaunch(KernelTimer* timer, const char* kind, hipStream_t stream, bool several_kernels = false)
      : t(timer), s(stream), markers(several_kernels), outer(t_launch_events) {
    if (t) on = t->begin(kind, s, markers, &ev.start, &ev.stop);
    if (on && !markers) t_launch_events = &ev;
  }
  ~TimedLaunch() {
    if (on && !markers) t_launch_events = outer;
    if (on) t->end(s, markers, ev.start, ev.stop, markers ? 1 : ev.launched);
  }
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;
};

// kernel<<<grid, block, shmem, s>>>(args...) through the runtime's launch
// call; inside a TimedLaunch scope the first such launch carries the scope's
// events.  Errors are left for hipGetLastError, as with <<<>>>.
template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                   Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals{static_cast<KArgs>(args)...};
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&ptrs](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  hipEvent_t a = nullptr, b = nullptr;
  if (LaunchEvents* ev = t_launch_events) {
    if (ev->launched++ == 0) {
      a = ev->start;
      b = ev->stop;
    }
  }
  const void* fn = reinterpret_cast<const void*>(kernel);
  if (a)
    (void)hipExtLaunchKernel(fn, grid, block, ptrs, shmem, s, a, b, 0);
  else
    (void)hipLaunchKernel(fn, grid, block, ptrs, shmem, s);
}

// ----- selection (select.hip) -----
hipError_t launch_select(const float* score, int32_t* age, int B, int N, int k, int G, int rows_cap,
                         int32_t* idx, int32_t* k_eff, int32_t* n_forced, hipStream_t s);
// Selection fused with the last scoring step: the scores are formed from the
// per-token P, U and the per-block U partials (nblocks per episode), written
// to score_out, and selected on in the same kernel.
struct ScoreInputs {
  const float* mass;
  const float* surprise;
  const float* usum;
  int nblocks;
  float w_attn_norm, w_surprise;
  float* score_out;
};
hipError_t launch_select_scored(const ScoreInputs& si, int32_t* age, int B, int N, int k, int G, int rows_cap,
                                int32_t* idx, int32_t* k_eff, int32_t* n_forced, hipStream_t s);
// union rule: top n_attn by mass, top n_surprise by surprise, forced; k_eff = union size
hipError_t launch_select_union(const float* mass, const float* surprise, int32_t* age, int B, int N, int n_attn,
                               int n_surprise, int G, int32_t* idx, int32_t* k_eff, int32_t* n_forced,
                               hipStream_t s);
hipError_t launch_ages_from_set(const int32_t* idx_in, const int32_t* k_in, int B, int N, int rows_cap,
                                int32_t* idx_out, int32_t* k_out, int32_t* age, hipStream_t s);

// ----- scoring (score.hip) -----
struct ScorePlan {
  int chunk_keys, nchunks, comb_blocks;
  size_t ms_bytes, part_bytes, tok_bytes, usum_bytes;
};
ScorePlan plan_score(int B, int L, int H, int N, int A, bool bf16);
hipError_t launch_score_mass(bool bf16, const void* qa, const void* kc, int B, int L, int H, int N,
                             int A, int d, const ScorePlan& p, float2* ms, float* part,
                             hipStream_t s, KernelTimer* timer);
// per-token P (sum over L*H) and U, and per-block partial sums of U
hipError_t launch_score_partials(bool bf16, const float* part, int LH, const float* mass_in, const void* z,
                                 const void* zref, int B, int N, int d, const ScorePlan& p, float* mass_tmp,
                                 float* surprise_tmp, float* usum, hipStream_t s, KernelTimer* timer);
// score = w_a P/(LHA) + w_s U / sum(U)
hipError_t launch_score_finish(const float* mass_tmp, const float* surprise_tmp, const float* usum, int B, int N,
                               float w_attn_norm, float w_surprise, const ScorePlan& p, float* score,
                               float* mass_out, float* surprise_out, hipStream_t s, KernelTimer* timer);

// ----- row kernels (rows.hip) -----
// Side job of the first row kernel of a call: zero two int arrays (the
// arrival counters of the split GEMM / attention), so no extra launch is needed.
struct ZeroJob {
  int* p0 = nullptr;
  int n0 = 0;
  int* p1 = nullptr;
  int n1 = 0;
};
// x[b*rows_cap + r] = float(z[b, idx[b,r]]), zref[b, idx] = z[b, idx]
// (idx == nullptr: identity, rows = all N tokens; age (nullable) <- 0).
hipError_t launch_gather(bool bf16, const void* z, void* zref, const int32_t* idx, const int32_t* k_eff,
                         int B, int N, int d, int rows_cap, float* x, int32_t* age_zero, const ZeroJob& zj,
                         hipStream_t s, KernelTimer* timer);
// gather fused with the first modulated LayerNorm (d <= 4096): also writes
// h = act(LN(x) * (1 + scale) + shift)
hipError_t launch_gather_ln(bool bf16, const void* z, void* zref, const int32_t* idx, const int32_t* k_eff, int B,
                            int N, int d, int rows_cap, float* x, int32_t* age_zero, const void* shift,
                            const void* scale, float eps, void* h, const ZeroJob& zj, hipStream_t s,
                            KernelTimer* timer);
// h[m] = act(LN(x_in[m]) * (1 + scale) + shift) for valid rows (shift == scale
// == nullptr: act(LN(x_in[m]))).
hipError_t launch_ln_mod(bool bf16, const float* x, const void* shift, const void* scale, int B,
                         int rows_cap, const int32_t* k_eff, int d, float eps, void* h, const ZeroJob& zj,
                         hipStream_t s, KernelTimer* timer);

// ----- GEMM (gemm.hip) -----
// EPI_RESID_OUT and EPI_RESID_DOWN share one epilogue; they are separate
// instances so profilers tell the two projections apart.
// EPI_KV: the text keys/values (cols [0,d) -> k_cache row, [d,2d) -> v_cache row);
// EPI_STORE: act(acc + bias) to g_out; EPI_RESID_PLAIN: out = in + (acc + bias).
enum GemmEpi {
  EPI_QKV = 0, EPI_RESID_OUT = 1, EPI_GELU = 2, EPI_RESID_DOWN = 3, EPI_KV = 4, EPI_STORE = 5, EPI_RESID_PLAIN = 6
};
struct GemmArgs {
  const void* a;        // [M, K] act, row-major
  const void* w;        // [Nout, K] act, row-major (linear-layer layout)
  const void* bias;     // [Nout] act
  int M, Nout, K;       // M = B * rows_cap
  int rows_cap;         // rows per episode
  const int32_t* k_eff; // nullable: valid rows per episode
  int rows_lo;          // host-side lower bound on k_eff[b] (the tile shape is chosen for it; 0 = unknown)
  // EPI_QKV: out cols [0,d) -> q_out[m, c]; [d,2d) -> k cache row; [2d,3d) -> v cache row
  void* q_out;
  void* k_cache;        // [B, N, d] act (this layer)
  void* v_cache;
  const int32_t* idx;   // nullable: [B, N] token of each row (identity when null)
  int n_tokens, d_model;
  // EPI_RESID_*: out[m, c] = in[m, c] + gate[c] * (acc + bias[c])   (f32)
  const float* resid_in;
  float* resid_out;
  const void* gate;     // [Nout] act
  // EPI_GELU: g[m, c] = act(gelu(acc + bias[c]))
  void* g_out;
  // scratch of the work-balanced bf16 path (nullable: plain tiles are used)
  float* sk_partial;        // f32 partial tiles of split output tiles
  size_t sk_partial_bytes;  // its size (bounds the number of pieces)
  int* sk_counters;         // per-tile arrival counters, zero between launches
  int parts;                // pieces per tile of the split-K path with a separate reduction (set by launch_gemm;
                            // -S: at most S, the count derived from k_eff on the device)
  // EPI_RESID_* (optional): the LayerNorm that follows, h = act(LN(out)(1 + scale) + shift) (no
  // modulation when shift is null), done in the same pass where the schedule holds whole rows
  void* ln_out;             // [M, d] act; null: no LayerNorm here
  const void* ln_shift;     // [d] act, nullable
  const void* ln_scale;     // [d] act
  float ln_eps;
};
// *ln_done (nullable) tells whether the LayerNorm asked for in g.ln_out was done.
hipError_t launch_gemm(bool bf16, GemmEpi epi, const GemmArgs& g, hipStream_t s, KernelTimer* timer,
                       bool* ln_done = nullptr);

// Scratch of the work-balanced bf16 GEMM for one layer's four projections.
struct GemmScratch {
  size_t partial_bytes, counter_bytes;
  int counters;
};
GemmScratch gemm_scratch(int B, int rows_cap, int d, int F);

// ----- attention (attention.hip) -----
struct AttnArgs {
  const void* q;        // [B*rows_cap, d] act
  const void* k_cache;  // [B, N, d] act
  const void* v_cache;
  void* o;              // [B*rows_cap, d] act
  int B, N, H, dh, d, rows_cap;
  const int32_t* k_eff;
  // scratch of the key-split bf16 path (nullable: one workgroup per query tile)
  float* part;          // [slots, kAttnPartFloats] partial (o, m, l) per piece
  int* counters;        // per-unit arrival counters, zero between launches
  int slots;
};
hipError_t launch_attention(bool bf16, const AttnArgs& a, hipStream_t s, KernelTimer* timer);

// Scratch of the key-split attention for B episodes of rows_cap rows and H heads.
#ifndef WAMC_ATTN_GROUPS
#define WAMC_ATTN_GROUPS 2
#endif
// two partial slots per resident workgroup (256 per CU-round with 8-wave
// workgroups, 512 with 4-wave ones)
constexpr int kAttnSlotsMax = 512 * (WAMC_ATTN_GROUPS == 1 ? 2 : 1);
constexpr int kAttnPartFloats = 128 * 128 + 2 * 256;   // o (128 queries x 128 dh) + m, l per lane
struct AttnScratch {
  size_t part_bytes, counter_bytes;
  int slots, counters;
};
AttnScratch attn_scratch(int B, int rows_cap, int H);

}  // namespace wamc
