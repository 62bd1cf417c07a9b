// C ABI of libwamc: argument validation, workspace layout, launch sequencing
// and the optional per-kernel timer.  See include/wamc.h for the contract.
#include "../../include/wamc.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

using namespace wamc;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("WAMC_DEBUG_SYNC");
    return e && e[0] && std::strcmp(e, "0") != 0;
  }();
  return on;
}

// ---------------------------------------------------------------------------
// kernel timer
// ---------------------------------------------------------------------------

class EventTimer final : public KernelTimer {
 public:
  struct Kind {
    std::string name;
    int launches = 0;
    double ms = 0.0;
  };
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };

  std::mutex mu;
  bool enabled = false;
  std::vector<Kind> kinds;
  std::vector<Rec> open;      // scopes begun, not yet ended
  std::vector<Rec> pending;   // ended, events not yet read
  std::vector<hipEvent_t> pool;

  hipEvent_t get_event() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }

  bool begin(const char* kind, hipStream_t s, bool markers, hipEvent_t* start, hipEvent_t* stop) override {
    std::lock_guard<std::mutex> lk(mu);
    hipEvent_t a = get_event();
    hipEvent_t b = a ? get_event() : nullptr;
    if (!a || !b || (markers && hipEventRecord(a, s) != hipSuccess)) {
      if (a) pool.push_back(a);
      if (b) pool.push_back(b);
      return false;
    }
    int k = -1;
    for (size_t i = 0; i < kinds.size(); ++i)
      if (kinds[i].name == kind) k = static_cast<int>(i);
    if (k < 0) {
      kinds.push_back(Kind{kind, 0, 0.0});
      k = static_cast<int>(kinds.size()) - 1;
    }
    open.push_back(Rec{k, a, b});
    *start = a;
    *stop = b;
    return true;
  }

  void end(hipStream_t s, bool markers, hipEvent_t start, hipEvent_t stop, int launched) override {
    std::lock_guard<std::mutex> lk(mu);
    for (size_t i = open.size(); i-- > 0;) {
      if (open[i].a != start) continue;
      const Rec r = open[i];
      open.erase(open.begin() + static_cast<long>(i));
      // a scope whose kernel never launched (or that launched more than the
      // one kernel the events describe) leaves no record
      if (launched == 1 && (!markers || hipEventRecord(stop, s) == hipSuccess)) {
        pending.push_back(r);
      } else {
        pool.push_back(r.a);
        pool.push_back(r.b);
      }
      return;
    }
  }

  void resolve() {
    std::lock_guard<std::mutex> lk(mu);
    for (const Rec& r : pending) {
      float ms = 0.f;
      if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
        kinds[r.kind].launches += 1;
        kinds[r.kind].ms += ms;
      }
      pool.push_back(r.a);
      pool.push_back(r.b);
    }
    pending.clear();
  }
};

EventTimer& timer_registry() {
  static EventTimer* t = new EventTimer();   // lives until process exit
  return *t;
}

KernelTimer* active_timer() {
  EventTimer& t = timer_registry();
  return t.enabled ? &t : nullptr;
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                        \
  do {                                                                        \
    if (!(p)) return fail(WAMC_ERR_ARG, "%s: '%s' must not be NULL", fn, #p); \
    if (!aligned(p)) return fail(WAMC_ERR_ALIGN, "%s: '%s' is not 16-byte aligned", fn, #p); \
  } while (0)

#define OPT_PTR(p)                                                            \
  do {                                                                        \
    if ((p) && !aligned(p)) return fail(WAMC_ERR_ALIGN, "%s: '%s' is not 16-byte aligned", fn, #p); \
  } while (0)

int check_dims(const char* fn, const wamc_dims* d) {
  if (!d) return fail(WAMC_ERR_ARG, "%s: dims is NULL", fn);
  if (d->batch < 1 || d->n_layers < 1 || d->d_model < 1 || d->n_heads < 1 || d->head_dim < 1 ||
      d->d_ffn < 1 || d->n_tokens < 1 || d->n_action < 1)
    return fail(WAMC_ERR_ARG, "%s: every size must be >= 1", fn);
  if (static_cast<long long>(d->n_heads) * d->head_dim != d->d_model)
    return fail(WAMC_ERR_ARG, "%s: d_model (%d) != n_heads (%d) * head_dim (%d)", fn, d->d_model,
                d->n_heads, d->head_dim);
  if (d->dtype != WAMC_FP32 && d->dtype != WAMC_BF16)
    return fail(WAMC_ERR_ARG, "%s: unknown dtype %d", fn, d->dtype);
  if (d->age_bound < 0) return fail(WAMC_ERR_ARG, "%s: age_bound must be >= 0", fn);
  if (!(d->ln_eps > 0.f) || !std::isfinite(d->ln_eps))
    return fail(WAMC_ERR_ARG, "%s: ln_eps must be a positive finite number", fn);
  if (!std::isfinite(d->w_attn) || !std::isfinite(d->w_surprise))
    return fail(WAMC_ERR_ARG, "%s: score weights must be finite", fn);
  const long long rows = static_cast<long long>(d->batch) * d->n_tokens;
  if (rows > (1ll << 30) || static_cast<long long>(d->d_ffn) > (1 << 22) ||
      static_cast<long long>(d->d_model) > (1 << 20) || rows * d->d_model > (1ll << 40))
    return fail(WAMC_ERR_ARG, "%s: sizes exceed the supported range", fn);
  if (d->d_model % 8 || d->d_ffn % 8)
    return fail(WAMC_ERR_UNSUPPORTED, "%s: d_model and d_ffn must be multiples of 8", fn);
  if (d->dtype == WAMC_BF16 && d->head_dim != 128)
    return fail(WAMC_ERR_UNSUPPORTED, "%s: the bf16 path is built for head_dim 128 (got %d)", fn, d->head_dim);
  if (d->dtype == WAMC_FP32 && d->head_dim > 128)
    return fail(WAMC_ERR_UNSUPPORTED, "%s: the fp32 path supports head_dim <= 128 (got %d)", fn, d->head_dim);
  if (d->n_text < 0 || d->n_text > (1 << 20)) return fail(WAMC_ERR_ARG, "%s: n_text must be in [0, 2^20]", fn);
  return WAMC_OK;
}

int check_rows_cap(const char* fn, const wamc_dims* d, int32_t rows_cap) {
  if (rows_cap < 1 || rows_cap > d->n_tokens)
    return fail(WAMC_ERR_ARG, "%s: rows_cap (%d) must be in [1, N=%d]", fn, rows_cap, d->n_tokens);
  return WAMC_OK;
}

int check_action(const char* fn, const wamc_dims* d) {
  if (d->dtype == WAMC_BF16 && d->n_action > 128)
    return fail(WAMC_ERR_UNSUPPORTED, "%s: the bf16 attention-mass kernel supports n_action <= 128", fn);
  if (d->dtype == WAMC_FP32 && d->n_action > 4096)
    return fail(WAMC_ERR_UNSUPPORTED, "%s: the fp32 attention-mass kernel supports n_action <= 4096", fn);
  return WAMC_OK;
}

int check_device(const char* fn) {
  static std::mutex mu;
  static std::map<int, int> known;   // device -> 1 ok, 0 not gfx950
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(WAMC_ERR_DEVICE, "%s: no HIP device", fn);
  std::lock_guard<std::mutex> lk(mu);
  auto it = known.find(dev);
  if (it == known.end()) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return fail(WAMC_ERR_DEVICE, "%s: cannot query device", fn);
    const int ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    it = known.emplace(dev, ok).first;
  }
  if (!it->second) return fail(WAMC_ERR_UNSUPPORTED, "%s: libwamc is built for gfx950 only", fn);
  return WAMC_OK;
}

size_t act_size(const wamc_dims* d) { return d->dtype == WAMC_BF16 ? 2 : 4; }

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Workspace: score region first (independent of rows_cap), then row buffers.
struct WsLayout {
  ScorePlan sp;
  size_t ms, part, mass_tmp, surp_tmp, usum, score_tmp;   // score region
  size_t x, hbuf, qbuf, gbuf;                              // row region
  GemmScratch gs;                                          // work-balanced GEMM scratch (bf16)
  size_t sk_partial, sk_counters;
  AttnScratch as;                                          // key-split attention scratch (bf16)
  size_t at_part, at_counters;
  size_t score_end, total;
};

WsLayout ws_layout(const wamc_dims* d, int32_t rows_cap) {
  WsLayout w;
  const bool bf16 = d->dtype == WAMC_BF16;
  w.sp = plan_score(d->batch, d->n_layers, d->n_heads, d->n_tokens, d->n_action, bf16);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  w.ms = take(w.sp.ms_bytes);
  w.part = take(w.sp.part_bytes);
  w.mass_tmp = take(w.sp.tok_bytes);
  w.surp_tmp = take(w.sp.tok_bytes);
  w.usum = take(w.sp.usum_bytes);
  w.score_tmp = take(w.sp.tok_bytes);
  w.score_end = off;
  const size_t rows = static_cast<size_t>(d->batch) * (rows_cap > 0 ? rows_cap : 0);
  w.x = take(rows * d->d_model * sizeof(float));
  w.hbuf = take(rows * d->d_model * act_size(d));
  w.qbuf = take(rows * d->d_model * act_size(d));
  w.gbuf = take(rows * d->d_ffn * act_size(d));
  w.gs = bf16 ? gemm_scratch(d->batch, rows_cap, d->d_model, d->d_ffn) : GemmScratch{};
  w.sk_partial = take(w.gs.partial_bytes);
  w.sk_counters = take(w.gs.counter_bytes);
  w.as = bf16 && d->head_dim == 128 ? attn_scratch(d->batch, rows_cap, d->n_heads) : AttnScratch{};
  w.at_part = take(w.as.part_bytes);
  w.at_counters = take(w.as.counter_bytes);
  w.total = off;
  return w;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

const void* offset(const void* p, size_t elems, size_t esize) {
  return static_cast<const char*>(p) + elems * esize;
}

int hip_status(const char* fn, hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return fail(WAMC_ERR_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(WAMC_ERR_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  }
  return WAMC_OK;
}

int check_layer_w(const char* fn, const wamc_layer_w* w, int n_text = 0) {
  if (!w) return fail(WAMC_ERR_ARG, "%s: layer weights are NULL", fn);
  if (n_text > 0) {
    REQUIRE_PTR(w->w_qc);
    REQUIRE_PTR(w->b_qc);
    REQUIRE_PTR(w->w_kvc);
    REQUIRE_PTR(w->b_kvc);
    REQUIRE_PTR(w->w_oc);
    REQUIRE_PTR(w->b_oc);
    REQUIRE_PTR(w->text_k);
    REQUIRE_PTR(w->text_v);
  }
  REQUIRE_PTR(w->w_qkv);
  REQUIRE_PTR(w->b_qkv);
  REQUIRE_PTR(w->w_o);
  REQUIRE_PTR(w->b_o);
  REQUIRE_PTR(w->w_1);
  REQUIRE_PTR(w->b_1);
  REQUIRE_PTR(w->w_2);
  REQUIRE_PTR(w->b_2);
  REQUIRE_PTR(w->mod);
  return WAMC_OK;
}

// The arrival counters of the split GEMM / attention start every call at zero
// (the kernels leave them so); the first row kernel of the call clears them.
ZeroJob counter_clear(void* ws, const WsLayout& L) {
  ZeroJob z;
  if (L.gs.counters > 0) {
    z.p0 = at<int>(ws, L.sk_counters);
    z.n0 = L.gs.counters;
  }
  if (L.as.counters > 0) {
    z.p1 = at<int>(ws, L.at_counters);
    z.n1 = L.as.counters;
  }
  return z;
}

// One layer on rows [b*rows_cap, b*rows_cap + k_eff[b]): reads x_in, writes
// x_out (may alias x_in).
// rows_lo: a lower bound on every k_eff[b] known on the host (0 when unknown),
// from which the GEMM tile shape is chosen.
// h1_ready: the layer's first modulated LayerNorm is already in the h buffer.
// next_shift1 / next_scale1 (nullable): the next layer's first modulation;
// when the MLP down projection can produce that LayerNorm in its own pass it
// does, and *next_h1_ready says so.
hipError_t run_layer(const wamc_dims* d, const wamc_layer_w* w, const float* x_in, float* x_out,
                     const int32_t* idx, const int32_t* k_eff, int32_t rows_cap, int32_t rows_lo, void* kc,
                     void* vc, void* ws, const WsLayout& L, hipStream_t s, bool h1_ready = false,
                     const ZeroJob& zj = ZeroJob{}, const void* next_shift1 = nullptr,
                     const void* next_scale1 = nullptr, bool* next_h1_ready = nullptr) {
  if (next_h1_ready) *next_h1_ready = false;
  const bool bf16 = d->dtype == WAMC_BF16;
  const size_t es = act_size(d);
  const int D = d->d_model, F = d->d_ffn, B = d->batch;
  KernelTimer* tm = active_timer();
  void* hbuf = at<char>(ws, L.hbuf);
  void* qbuf = at<char>(ws, L.qbuf);
  void* gbuf = at<char>(ws, L.gbuf);
  const void* shift1 = offset(w->mod, 0 * D, es);
  const void* scale1 = offset(w->mod, 1 * D, es);
  const void* gate1 = offset(w->mod, 2 * D, es);
  const void* shift2 = offset(w->mod, 3 * D, es);
  const void* scale2 = offset(w->mod, 4 * D, es);
  const void* gate2 = offset(w->mod, 5 * D, es);
  const int M = B * rows_cap;
  hipError_t e;

  if (!h1_ready) {
    e = launch_ln_mod(bf16, x_in, shift1, scale1, B, rows_cap, k_eff, D, d->ln_eps, hbuf, zj, s, tm);
    if (e != hipSuccess) return e;
  }

  GemmArgs g{};
  g.rows_cap = rows_cap;
  g.k_eff = k_eff;
  g.rows_lo = k_eff ? rows_lo : rows_cap;
  g.M = M;
  g.n_tokens = d->n_tokens;
  g.d_model = D;
  g.idx = idx;
  if (L.gs.partial_bytes > 0) {
    g.sk_partial = at<float>(ws, L.sk_partial);
    g.sk_partial_bytes = L.gs.partial_bytes;
    g.sk_counters = at<int>(ws, L.sk_counters);
  }

  g.a = hbuf; g.w = w->w_qkv; g.bias = w->b_qkv; g.Nout = 3 * D; g.K = D;
  g.q_out = qbuf; g.k_cache = kc; g.v_cache = vc;
  e = launch_gemm(bf16, EPI_QKV, g, s, tm);
  if (e != hipSuccess) return e;

  AttnArgs at_{};
  at_.q = qbuf; at_.k_cache = kc; at_.v_cache = vc; at_.o = hbuf;
  at_.B = B; at_.N = d->n_tokens; at_.H = d->n_heads; at_.dh = d->head_dim; at_.d = D;
  at_.rows_cap = rows_cap; at_.k_eff = k_eff;
  if (L.as.slots > 0) {
    at_.part = at<float>(ws, L.at_part);
    at_.counters = at<int>(ws, L.at_counters);
    at_.slots = L.as.slots;
  }
  e = launch_attention(bf16, at_, s, tm);
  if (e != hipSuccess) return e;

  // The LayerNorm after each residual projection (the text query's plain one,
  // or adaLN-2) comes from the projection's own pass where its schedule holds
  // whole rows (ln_done), else from the LayerNorm kernel.
  g.a = hbuf; g.w = w->w_o; g.bias = w->b_o; g.Nout = D; g.K = D;
  g.resid_in = x_in; g.resid_out = x_out; g.gate = gate1;
  g.ln_out = hbuf; g.ln_eps = d->ln_eps;
  g.ln_shift = d->n_text > 0 ? nullptr : shift2;
  g.ln_scale = d->n_text > 0 ? nullptr : scale2;
  bool ln_done = false;
  e = launch_gemm(bf16, EPI_RESID_OUT, g, s, tm, &ln_done);
  g.ln_out = nullptr;
  if (e != hipSuccess) return e;

  if (d->n_text > 0) {
    // text cross-attention: Qc = LN(x) W_qc^T + b_qc; x += attn(Qc, K_t, V_t) W_oc^T + b_oc
    if (!ln_done) {
      e = launch_ln_mod(bf16, x_out, nullptr, nullptr, B, rows_cap, k_eff, D, d->ln_eps, hbuf, ZeroJob{}, s, tm);
      if (e != hipSuccess) return e;
    }
    g.a = hbuf; g.w = w->w_qc; g.bias = w->b_qc; g.Nout = D; g.K = D; g.g_out = qbuf;
    e = launch_gemm(bf16, EPI_STORE, g, s, tm);
    if (e != hipSuccess) return e;
    AttnArgs ca = at_;
    ca.k_cache = w->text_k; ca.v_cache = w->text_v; ca.N = d->n_text;
    e = launch_attention(bf16, ca, s, tm);
    if (e != hipSuccess) return e;
    g.a = hbuf; g.w = w->w_oc; g.bias = w->b_oc; g.Nout = D; g.K = D;
    g.resid_in = x_out; g.resid_out = x_out; g.gate = nullptr;
    g.ln_out = hbuf; g.ln_shift = shift2; g.ln_scale = scale2;
    e = launch_gemm(bf16, EPI_RESID_PLAIN, g, s, tm, &ln_done);
    g.ln_out = nullptr;
    if (e != hipSuccess) return e;
  }

  if (!ln_done) {
    e = launch_ln_mod(bf16, x_out, shift2, scale2, B, rows_cap, k_eff, D, d->ln_eps, hbuf, ZeroJob{}, s, tm);
    if (e != hipSuccess) return e;
  }

  g.a = hbuf; g.w = w->w_1; g.bias = w->b_1; g.Nout = F; g.K = D; g.g_out = gbuf;
  e = launch_gemm(bf16, EPI_GELU, g, s, tm);
  if (e != hipSuccess) return e;

  g.a = gbuf; g.w = w->w_2; g.bias = w->b_2; g.Nout = D; g.K = F;
  g.resid_in = x_out; g.resid_out = x_out; g.gate = gate2;
  if (next_shift1) {
    g.ln_out = hbuf; g.ln_shift = next_shift1; g.ln_scale = next_scale1;
  }
  return launch_gemm(bf16, EPI_RESID_DOWN, g, s, tm, next_h1_ready);
}

// Attention mass (unless supplied) and the per-token P, U partials.
hipError_t run_score_partials(const wamc_dims* d, const void* z, const void* zref, const void* q_act,
                              const void* k_cache, const float* mass_in, void* ws, const WsLayout& L,
                              hipStream_t s) {
  const bool bf16 = d->dtype == WAMC_BF16;
  KernelTimer* tm = active_timer();
  const int LH = d->n_layers * d->n_heads;
  float* part = at<float>(ws, L.part);
  if (!mass_in) {
    hipError_t e = launch_score_mass(bf16, q_act, k_cache, d->batch, d->n_layers, d->n_heads, d->n_tokens,
                                     d->n_action, d->d_model, L.sp, at<float2>(ws, L.ms), part, s, tm);
    if (e != hipSuccess) return e;
  }
  return launch_score_partials(bf16, part, LH, mass_in, z, zref, d->batch, d->n_tokens, d->d_model, L.sp,
                               at<float>(ws, L.mass_tmp), at<float>(ws, L.surp_tmp), at<float>(ws, L.usum), s, tm);
}

float attn_weight_norm(const wamc_dims* d) {
  return d->w_attn / (static_cast<float>(d->n_layers * d->n_heads) * static_cast<float>(d->n_action));
}

hipError_t run_score(const wamc_dims* d, const void* z, const void* zref, const void* q_act,
                     const void* k_cache, const float* mass_in, float* score, float* mass_out,
                     float* surprise_out, void* ws, const WsLayout& L, hipStream_t s) {
  hipError_t e = run_score_partials(d, z, zref, q_act, k_cache, mass_in, ws, L, s);
  if (e != hipSuccess) return e;
  return launch_score_finish(at<float>(ws, L.mass_tmp), at<float>(ws, L.surp_tmp), at<float>(ws, L.usum), d->batch,
                             d->n_tokens, attn_weight_norm(d), d->w_surprise, L.sp, score, mass_out, surprise_out, s,
                             active_timer());
}


// Gather the selected rows (fused with layer 0's first LayerNorm when d fits)
// and run every layer on them.
hipError_t run_refresh_rows(const wamc_dims* dims, const wamc_layer_w* layers, const void* z, void* zref,
                            void* k_cache, void* v_cache, const int32_t* idx, const int32_t* k_eff, float* layer_out,
                            int32_t rows_cap, int32_t rows_lo, void* ws, const WsLayout& L, hipStream_t s) {
  KernelTimer* tm = active_timer();
  const bool bf16 = dims->dtype == WAMC_BF16;
  const int B = dims->batch, N = dims->n_tokens, D = dims->d_model;
  float* x = at<float>(ws, L.x);
  const size_t es = act_size(dims);
  const bool fuse_ln = D <= 4096;
  hipError_t e;
  if (fuse_ln)
    e = launch_gather_ln(bf16, z, zref, idx, k_eff, B, N, D, rows_cap, x, nullptr, offset(layers[0].mod, 0, es),
                         offset(layers[0].mod, D, es), dims->ln_eps, at<char>(ws, L.hbuf), counter_clear(ws, L), s, tm);
  else
    e = launch_gather(bf16, z, zref, idx, k_eff, B, N, D, rows_cap, x, nullptr, counter_clear(ws, L), s, tm);
  const size_t layer_elems = static_cast<size_t>(B) * N * D;
  const size_t out_elems = static_cast<size_t>(B) * rows_cap * D;
  bool h1 = fuse_ln;
  for (int l = 0; l < dims->n_layers && e == hipSuccess; ++l) {
    const float* xin = (layer_out && l > 0) ? layer_out + (l - 1) * out_elems : x;
    float* xout = layer_out ? layer_out + l * out_elems : x;
    void* kc = static_cast<char*>(k_cache) + l * layer_elems * es;
    void* vc = static_cast<char*>(v_cache) + l * layer_elems * es;
    const bool next = l + 1 < dims->n_layers;
    e = run_layer(dims, &layers[l], xin, xout, idx, k_eff, rows_cap, rows_lo, kc, vc, ws, L, s, h1, ZeroJob{},
                  next ? offset(layers[l + 1].mod, 0, es) : nullptr, next ? offset(layers[l + 1].mod, D, es) : nullptr,
                  &h1);
  }
  return e;
}

}  // namespace

namespace wamc {
// The thread's error detail for entry points defined in other files.
int api_fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}
}  // namespace wamc

// ===========================================================================
// exported API
// ===========================================================================

extern "C" {

int wamc_version(void) { return WAMC_VERSION; }

const char* wamc_status_string(int status) {
  switch (status) {
    case WAMC_OK: return "ok";
    case WAMC_ERR_ARG: return "invalid argument";
    case WAMC_ERR_UNSUPPORTED: return "unsupported configuration";
    case WAMC_ERR_WORKSPACE: return "workspace too small";
    case WAMC_ERR_ALIGN: return "pointer not 16-byte aligned";
    case WAMC_ERR_DEVICE: return "HIP device error";
    default: return "unknown status";
  }
}

const char* wamc_last_error(void) { return g_last_error.c_str(); }

int wamc_workspace_bytes(const wamc_dims* dims, int32_t rows_cap, size_t* bytes) {
  const char* fn = "wamc_workspace_bytes";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  if (!bytes) return fail(WAMC_ERR_ARG, "%s: bytes is NULL", fn);
  if (rows_cap < 0 || rows_cap > dims->n_tokens)
    return fail(WAMC_ERR_ARG, "%s: rows_cap (%d) must be in [0, N=%d]", fn, rows_cap, dims->n_tokens);
  *bytes = ws_layout(dims, rows_cap).total;
  return WAMC_OK;
}

int wamc_score(const wamc_dims* dims, const void* z, const void* zref, const void* q_act,
               const void* k_cache, const float* mass_in, float* score, float* mass_out,
               float* surprise_out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "wamc_score";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(z);
  REQUIRE_PTR(zref);
  REQUIRE_PTR(score);
  OPT_PTR(mass_in);
  OPT_PTR(mass_out);
  OPT_PTR(surprise_out);
  if (!mass_in) {
    REQUIRE_PTR(q_act);
    REQUIRE_PTR(k_cache);
    if ((st = check_action(fn, dims))) return st;
  }
  const WsLayout L = ws_layout(dims, 0);
  if (!ws || ws_bytes < L.score_end)
    return fail(WAMC_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.score_end);
  OPT_PTR(ws);
  if ((st = check_device(fn))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(fn, run_score(dims, z, zref, q_act, k_cache, mass_in, score, mass_out, surprise_out, ws, L, s), s);
}

int wamc_select(const wamc_dims* dims, const float* score, int32_t* age, int32_t k, int32_t rows_cap,
                int32_t* idx, int32_t* k_eff, int32_t* n_forced, void* stream) {
  const char* fn = "wamc_select";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(score);
  REQUIRE_PTR(age);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(k_eff);
  OPT_PTR(n_forced);
  if (k < 0 || k > dims->n_tokens) return fail(WAMC_ERR_ARG, "%s: k (%d) must be in [0, N=%d]", fn, k, dims->n_tokens);
  if ((st = check_rows_cap(fn, dims, rows_cap))) return st;
  if (rows_cap < k) return fail(WAMC_ERR_ARG, "%s: rows_cap (%d) < k (%d)", fn, rows_cap, k);
  if ((st = check_device(fn))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  KernelTimer* tm = active_timer();
  hipError_t e;
  {
    TimedLaunch t(tm, "select", s);
    e = launch_select(score, age, dims->batch, dims->n_tokens, k, dims->age_bound, rows_cap, idx, k_eff, n_forced, s);
  }
  return hip_status(fn, e, s);
}

int wamc_gather(const wamc_dims* dims, const void* z, void* zref, const int32_t* idx, const int32_t* k_eff,
                int32_t rows_cap, float* x, void* stream) {
  const char* fn = "wamc_gather";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(z);
  REQUIRE_PTR(zref);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(k_eff);
  REQUIRE_PTR(x);
  if ((st = check_rows_cap(fn, dims, rows_cap))) return st;
  if ((st = check_device(fn))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(fn, launch_gather(dims->dtype == WAMC_BF16, z, zref, idx, k_eff, dims->batch, dims->n_tokens,
                                      dims->d_model, rows_cap, x, nullptr, ZeroJob{}, s, active_timer()), s);
}

int wamc_refresh_layer(const wamc_dims* dims, int32_t layer, const wamc_layer_w* w, float* x,
                       const int32_t* idx, const int32_t* k_eff, int32_t rows_cap, void* k_cache_l,
                       void* v_cache_l, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "wamc_refresh_layer";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  if (layer < 0 || layer >= dims->n_layers)
    return fail(WAMC_ERR_ARG, "%s: layer %d out of range [0, %d)", fn, layer, dims->n_layers);
  if ((st = check_layer_w(fn, w, dims->n_text))) return st;
  REQUIRE_PTR(x);
  REQUIRE_PTR(k_cache_l);
  REQUIRE_PTR(v_cache_l);
  OPT_PTR(idx);
  OPT_PTR(k_eff);
  if ((st = check_rows_cap(fn, dims, rows_cap))) return st;
  const WsLayout L = ws_layout(dims, rows_cap);
  if (!ws || ws_bytes < L.total) return fail(WAMC_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  OPT_PTR(ws);
  if ((st = check_device(fn))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(fn, run_layer(dims, w, x, x, idx, k_eff, rows_cap, 0, k_cache_l, v_cache_l, ws, L, s, false,
                                  counter_clear(ws, L)), s);
}

int wamc_prefill_chunk(const wamc_dims* dims, const wamc_layer_w* layers, const void* z, void* zref,
                       const void* q_act, const float* mass_in, void* k_cache, void* v_cache, int32_t* age,
                       int32_t k, const int32_t* idx_override, const int32_t* k_eff_override, int32_t* idx_out,
                       int32_t* k_eff_out, float* score_out, float* layer_out, int32_t rows_cap, void* ws,
                       size_t ws_bytes, void* stream) {
  const char* fn = "wamc_prefill_chunk";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  if (!layers) return fail(WAMC_ERR_ARG, "%s: layers is NULL", fn);
  for (int l = 0; l < dims->n_layers; ++l)
    if ((st = check_layer_w(fn, &layers[l], dims->n_text))) return st;
  REQUIRE_PTR(z);
  REQUIRE_PTR(zref);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(age);
  REQUIRE_PTR(idx_out);
  REQUIRE_PTR(k_eff_out);
  OPT_PTR(score_out);
  OPT_PTR(layer_out);
  OPT_PTR(mass_in);
  if (k < 0 || k > dims->n_tokens) return fail(WAMC_ERR_ARG, "%s: k (%d) must be in [0, N=%d]", fn, k, dims->n_tokens);
  if ((st = check_rows_cap(fn, dims, rows_cap))) return st;
  if (rows_cap < k) return fail(WAMC_ERR_ARG, "%s: rows_cap (%d) < k (%d)", fn, rows_cap, k);
  if (!idx_override) {
    // With G >= 1 a forced token was not refreshed in the previous chunk,
    // which refreshed at least k tokens, so at most N - k are forced (all N
    // when G = 0).  A smaller capacity could leave forced tokens out.
    const int forced_max = dims->age_bound == 0 ? dims->n_tokens : dims->n_tokens - k;
    if (rows_cap < forced_max)
      return fail(WAMC_ERR_ARG,
                  "%s: rows_cap (%d) < %d, the most tokens the age bound can force (N - k, or N when G = 0): "
                  "forced tokens would be left out", fn, rows_cap, forced_max);
  }
  if (idx_override) {
    OPT_PTR(idx_override);
    if (!k_eff_override) return fail(WAMC_ERR_ARG, "%s: idx_override needs k_eff_override", fn);
  } else if (!mass_in) {
    REQUIRE_PTR(q_act);
    if ((st = check_action(fn, dims))) return st;
  }
  const WsLayout L = ws_layout(dims, rows_cap);
  if (!ws || ws_bytes < L.total) return fail(WAMC_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  OPT_PTR(ws);
  if ((st = check_device(fn))) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  KernelTimer* tm = active_timer();
  const int B = dims->batch, N = dims->n_tokens;
  hipError_t e;
  if (idx_override) {
    TimedLaunch t(tm, "ages_from_set", s, /*several_kernels=*/true);
    e = launch_ages_from_set(idx_override, k_eff_override, B, N, rows_cap, idx_out, k_eff_out, age, s);
  } else {
    // scoring's last step (sum of U, the weighted sum) runs inside the selection kernel
    e = run_score_partials(dims, z, zref, q_act, k_cache, mass_in, ws, L, s);
    if (e == hipSuccess) {
      ScoreInputs si;
      si.mass = at<float>(ws, L.mass_tmp);
      si.surprise = at<float>(ws, L.surp_tmp);
      si.usum = at<float>(ws, L.usum);
      si.nblocks = L.sp.comb_blocks;
      si.w_attn_norm = attn_weight_norm(dims);
      si.w_surprise = dims->w_surprise;
      si.score_out = score_out ? score_out : at<float>(ws, L.score_tmp);
      TimedLaunch t(tm, "select", s);
      e = launch_select_scored(si, age, B, N, k, dims->age_bound, rows_cap, idx_out, k_eff_out, nullptr, s);
    }
  }
  if (e != hipSuccess) return hip_status(fn, e, s);
  // k_eff = max(k, forced) >= k when the library selects; a supplied set's size is device data
  return hip_status(fn, run_refresh_rows(dims, layers, z, zref, k_cache, v_cache, idx_out, k_eff_out, layer_out,
                                         rows_cap, idx_override ? 0 : k, ws, L, s), s);
}

int wamc_select_union(const wamc_dims* dims, const float* mass, const float* surprise, int32_t* age,
                      int32_t n_attn, int32_t n_surprise, int32_t* idx, int32_t* k_eff, int32_t* n_forced,
                      void* stream) {
  const char* fn = "wamc_select_union";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  REQUIRE_PTR(mass);
  REQUIRE_PTR(surprise);
  REQUIRE_PTR(age);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(k_eff);
  OPT_PTR(n_forced);
  const int N = dims->n_tokens;
  if (n_attn < 0 || n_attn > N || n_surprise < 0 || n_surprise > N)
    return fail(WAMC_ERR_ARG, "%s: n_attn (%d) and n_surprise (%d) must be in [0, N=%d]", fn, n_attn, n_surprise, N);
  if ((st = check_device(fn))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    TimedLaunch t(active_timer(), "select", s);
    e = launch_select_union(mass, surprise, age, dims->batch, N, n_attn, n_surprise, dims->age_bound, idx, k_eff,
                            n_forced, s);
  }
  return hip_status(fn, e, s);
}

int wamc_prefill_chunk_union(const wamc_dims* dims, const wamc_layer_w* layers, const void* z, void* zref,
                             const void* q_act, const float* mass_in, void* k_cache, void* v_cache,
                             int32_t* age, int32_t n_attn, int32_t n_surprise, int32_t* idx_out,
                             int32_t* k_eff_out, float* layer_out, int32_t rows_cap, void* ws,
                             size_t ws_bytes, void* stream) {
  const char* fn = "wamc_prefill_chunk_union";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  if (!layers) return fail(WAMC_ERR_ARG, "%s: layers is NULL", fn);
  for (int l = 0; l < dims->n_layers; ++l)
    if ((st = check_layer_w(fn, &layers[l], dims->n_text))) return st;
  REQUIRE_PTR(z);
  REQUIRE_PTR(zref);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(age);
  REQUIRE_PTR(idx_out);
  REQUIRE_PTR(k_eff_out);
  OPT_PTR(layer_out);
  OPT_PTR(mass_in);
  const int N = dims->n_tokens;
  if (n_attn < 0 || n_attn > N || n_surprise < 0 || n_surprise > N)
    return fail(WAMC_ERR_ARG, "%s: n_attn (%d) and n_surprise (%d) must be in [0, N=%d]", fn, n_attn, n_surprise, N);
  if (rows_cap != N) return fail(WAMC_ERR_ARG, "%s: rows_cap (%d) must be N (%d)", fn, rows_cap, N);
  if (!mass_in) {
    REQUIRE_PTR(q_act);
    if ((st = check_action(fn, dims))) return st;
  }
  const WsLayout L = ws_layout(dims, rows_cap);
  if (!ws || ws_bytes < L.total) return fail(WAMC_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  OPT_PTR(ws);
  if ((st = check_device(fn))) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = run_score_partials(dims, z, zref, q_act, k_cache, mass_in, ws, L, s);
  if (e == hipSuccess) {
    TimedLaunch t(active_timer(), "select", s);
    e = launch_select_union(at<float>(ws, L.mass_tmp), at<float>(ws, L.surp_tmp), age, dims->batch, N, n_attn,
                            n_surprise, dims->age_bound, idx_out, k_eff_out, nullptr, s);
  }
  if (e != hipSuccess) return hip_status(fn, e, s);
  // the union holds at least the larger of the two budgets
  return hip_status(fn, run_refresh_rows(dims, layers, z, zref, k_cache, v_cache, idx_out, k_eff_out, layer_out,
                                         rows_cap, std::max(n_attn, n_surprise), ws, L, s), s);
}

int wamc_text_kv(const wamc_dims* dims, const wamc_layer_w* layers, const void* text, void* ws, size_t ws_bytes,
                 void* stream) {
  const char* fn = "wamc_text_kv";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  if (dims->n_text <= 0) return fail(WAMC_ERR_ARG, "%s: dims.n_text must be > 0", fn);
  if (!layers) return fail(WAMC_ERR_ARG, "%s: layers is NULL", fn);
  for (int l = 0; l < dims->n_layers; ++l)
    if ((st = check_layer_w(fn, &layers[l], dims->n_text))) return st;
  REQUIRE_PTR(text);
  const int T = dims->n_text;
  const WsLayout L = ws_layout(dims, std::min(T, dims->n_tokens));
  if (!ws || ws_bytes < L.total) return fail(WAMC_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  OPT_PTR(ws);
  if ((st = check_device(fn))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dims->dtype == WAMC_BF16;
  hipError_t e = hipSuccess;
  for (int l = 0; l < dims->n_layers && e == hipSuccess; ++l) {
    // one GEMM per layer: [B*T, d] x [2d, d]^T, K half -> text_k, V half -> text_v
    // (plain tiles: no split scratch, so the arrival counters are not needed)
    GemmArgs g{};
    g.a = text; g.w = layers[l].w_kvc; g.bias = layers[l].b_kvc;
    g.M = dims->batch * T; g.Nout = 2 * dims->d_model; g.K = dims->d_model;
    g.rows_cap = T; g.k_eff = nullptr; g.idx = nullptr;
    g.n_tokens = T; g.d_model = dims->d_model;
    g.k_cache = layers[l].text_k; g.v_cache = layers[l].text_v;
    e = launch_gemm(bf16, EPI_KV, g, s, active_timer());
  }
  return hip_status(fn, e, s);
}

int wamc_dense_prefill(const wamc_dims* dims, const wamc_layer_w* layers, const void* z, void* zref,
                       void* k_cache, void* v_cache, int32_t* age, float* layer_out, void* ws, size_t ws_bytes,
                       void* stream) {
  const char* fn = "wamc_dense_prefill";
  g_last_error.clear();
  int st = check_dims(fn, dims);
  if (st) return st;
  if (!layers) return fail(WAMC_ERR_ARG, "%s: layers is NULL", fn);
  for (int l = 0; l < dims->n_layers; ++l)
    if ((st = check_layer_w(fn, &layers[l], dims->n_text))) return st;
  REQUIRE_PTR(z);
  REQUIRE_PTR(zref);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(age);
  OPT_PTR(layer_out);
  const int N = dims->n_tokens;
  const WsLayout L = ws_layout(dims, N);
  if (!ws || ws_bytes < L.total) return fail(WAMC_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total);
  OPT_PTR(ws);
  if ((st = check_device(fn))) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  KernelTimer* tm = active_timer();
  const bool bf16 = dims->dtype == WAMC_BF16;
  const int B = dims->batch, D = dims->d_model;
  float* x = at<float>(ws, L.x);
  const size_t es = act_size(dims);
  const bool fuse_ln = D <= 4096;
  hipError_t e;
  if (fuse_ln)
    e = launch_gather_ln(bf16, z, zref, nullptr, nullptr, B, N, D, N, x, age, offset(layers[0].mod, 0, es),
                         offset(layers[0].mod, D, es), dims->ln_eps, at<char>(ws, L.hbuf), counter_clear(ws, L), s, tm);
  else
    e = launch_gather(bf16, z, zref, nullptr, nullptr, B, N, D, N, x, age, counter_clear(ws, L), s, tm);
  const size_t layer_elems = static_cast<size_t>(B) * N * D;
  bool h1 = fuse_ln;
  for (int l = 0; l < dims->n_layers && e == hipSuccess; ++l) {
    const float* xin = (layer_out && l > 0) ? layer_out + (l - 1) * layer_elems : x;
    float* xout = layer_out ? layer_out + l * layer_elems : x;
    void* kc = static_cast<char*>(k_cache) + l * layer_elems * es;
    void* vc = static_cast<char*>(v_cache) + l * layer_elems * es;
    const bool next = l + 1 < dims->n_layers;
    e = run_layer(dims, &layers[l], xin, xout, nullptr, nullptr, N, N, kc, vc, ws, L, s, h1, ZeroJob{},
                  next ? offset(layers[l + 1].mod, 0, es) : nullptr, next ? offset(layers[l + 1].mod, D, es) : nullptr,
                  &h1);
  }
  return hip_status(fn, e, s);
}

int wamc_timing_enable(int on) {
  EventTimer& t = timer_registry();
  t.resolve();
  std::lock_guard<std::mutex> lk(t.mu);
  t.enabled = on != 0;
  if (t.enabled) t.kinds.clear();
  return WAMC_OK;
}

int wamc_timing_count(void) {
  EventTimer& t = timer_registry();
  t.resolve();
  std::lock_guard<std::mutex> lk(t.mu);
  return static_cast<int>(t.kinds.size());
}

int wamc_timing_get(int i, const char** name, int32_t* launches, double* total_ms) {
  EventTimer& t = timer_registry();
  t.resolve();
  std::lock_guard<std::mutex> lk(t.mu);
  if (i < 0 || i >= static_cast<int>(t.kinds.size())) return fail(WAMC_ERR_ARG, "wamc_timing_get: index out of range");
  if (name) *name = t.kinds[i].name.c_str();
  if (launches) *launches = t.kinds[i].launches;
  if (total_ms) *total_ms = t.kinds[i].ms;
  return WAMC_OK;
}

}  // extern "C"
