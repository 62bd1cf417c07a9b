/*
 * wamc.h -- C ABI of libwamc, the MI355X (gfx950) library for the
 * staleness-bounded sparse KV-refresh prefill of a video-DiT observation
 * encoder, as described in "WAM-Cache: Staleness-Bounded KV Reuse for
 * Efficient World Action Models" (paperpeel 2610.11401).
 *
 * Each control chunk the video DiT keeps its layerwise K/V cache (§4.1
 * "Overview": per-token cached K/V for every layer, a reference embedding
 * stored at the token's last refresh, an age counter of consecutive reuses).
 * The library scores every visual token by the action expert's attention mass
 * over that token's cached keys plus latent surprise (§1, §4.2, §4.3), forces
 * every token whose age reached the bound into the refresh set (§4.4; the
 * RealtimeWAM page, App. D.3 "Recursive reuse": an age cap of G allows at
 * most G consecutive reuses), fills the set up to k by score, and recomputes
 * only those rows through every layer (§3 "Preliminaries": self-attention and
 * MLP with residuals; refreshed queries attend over all S_v cached and fresh
 * keys), writing their fresh K/V into the cache.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *   owned by the caller, 16-byte aligned, dense row-major with the shape
 *   given in the comments.  `stream` is a hipStream_t passed as void*
 *   (NULL = the default stream).  The library never allocates, frees or
 *   copies to or from the host, never changes the current device, and keeps
 *   no device state between calls.
 * - "act" tensors (weights, biases, modulation, z, zref, q_act, K/V cache)
 *   are float32 when dims.dtype == WAMC_FP32 and bfloat16 when
 *   dims.dtype == WAMC_BF16.  The residual stream x and every layer output
 *   are always float32.  Scores are float32; indices, ages and counts int32.
 * - B = dims.batch independent episodes share the weights; each has its own
 *   cache, ages, reference embeddings and refresh count (k_eff[b]).
 * - All calls are asynchronous on `stream`.  Arguments are validated on the
 *   host before anything is enqueued: a call that returns an error has
 *   enqueued nothing.  A fault inside a kernel surfaces at the caller's next
 *   synchronisation; with the environment variable WAMC_DEBUG_SYNC=1 every
 *   call synchronises its stream and reports WAMC_ERR_DEVICE instead.
 * - Row-indexed buffers hold, for episode b, rows [b*rows_cap, (b+1)*rows_cap);
 *   only the first k_eff[b] rows of an episode are meaningful.  Device-side
 *   counts are clamped to [0, rows_cap] and device-side token indices outside
 *   [0, N) are skipped, so malformed device inputs cannot write out of bounds.
 * - Results are deterministic: every reduction has a fixed order, so the same
 *   inputs give bitwise-identical outputs run after run.
 * - No C++ exception crosses this ABI; the only global state is a
 *   thread-local error string and the optional kernel-timing registry.
 */
#ifndef WAMC_H
#define WAMC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WAMC_VERSION 100  /* 1.0.0 */

enum wamc_status {
  WAMC_OK = 0,
  WAMC_ERR_ARG = 1,          /* null required pointer, inconsistent or out-of-range size */
  WAMC_ERR_UNSUPPORTED = 2,  /* dtype / head_dim / width not built, or not a gfx950 device */
  WAMC_ERR_WORKSPACE = 3,    /* workspace smaller than wamc_workspace_bytes() */
  WAMC_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned */
  WAMC_ERR_DEVICE = 5        /* a HIP call failed (launch error, or a fault seen under WAMC_DEBUG_SYNC) */
};

enum wamc_dtype { WAMC_FP32 = 0, WAMC_BF16 = 1 };

/* Model and method sizes.  Supported: d_model == n_heads * head_dim;
 * d_model and d_ffn multiples of 8; fp32: head_dim <= 128; bf16: head_dim ==
 * 128.  n_tokens (N) >= 1, n_action (A) >= 1 (used by wamc_score only),
 * age_bound (G) >= 0.  Range: batch * n_tokens <= 2^30, d_model <= 2^20,
 * d_ffn <= 2^22 and batch * n_tokens * d_model <= 2^40 (WAMC_ERR_ARG
 * beyond; the GEMM tiles address up to 256 rows of d_ffn elements with
 * 32-bit offsets from a 64-bit tile base). */
typedef struct {
  int32_t batch;        /* B episodes */
  int32_t n_layers;     /* L */
  int32_t d_model;      /* d */
  int32_t n_heads;      /* H */
  int32_t head_dim;     /* dh = d / H */
  int32_t d_ffn;        /* F */
  int32_t n_tokens;     /* N visual tokens per episode */
  int32_t n_action;     /* A action queries per layer */
  int32_t dtype;        /* enum wamc_dtype */
  int32_t age_bound;    /* G: a token whose age reached G is forced into the refresh set */
  float ln_eps;         /* LayerNorm epsilon (1e-6) */
  float w_attn;         /* weight of the attention-mass term of the score */
  float w_surprise;     /* weight of the latent-surprise term of the score */
  int32_t n_text;       /* T instruction tokens of the text cross-attention; 0 = the module has none */
} wamc_dims;

/* One layer's weights (act dtype), in the [out, in] layout of a linear map.
 * mod rows: shift1, scale1, gate1, shift2, scale2, gate2.
 * Text cross-attention (used when dims.n_text > 0, else may be NULL;
 * WAM-Cache §3: a module is self-attention, a cross-attention to keys and
 * values projected from the text embeddings, and an MLP, each with a
 * residual): its queries come from an unmodulated LayerNorm of the rows,
 * its residual is ungated.  text_k / text_v are this layer's keys and values
 * of the instruction, [B, T, d] act, caller-owned state written by
 * wamc_text_kv once per episode (they depend on the instruction only). */
typedef struct {
  const void *w_qkv, *b_qkv;   /* [3d, d], [3d]; output rows ordered Q, K, V; head h = cols [h*dh,(h+1)*dh) */
  const void *w_o, *b_o;       /* [d, d], [d] */
  const void *w_1, *b_1;       /* [F, d], [F] */
  const void *w_2, *b_2;       /* [d, F], [d] */
  const void *mod;             /* [6, d] */
  const void *w_qc, *b_qc;     /* [d, d], [d]   cross-attention queries */
  const void *w_kvc, *b_kvc;   /* [2d, d], [2d] cross-attention keys (rows 0..d-1) and values */
  const void *w_oc, *b_oc;     /* [d, d], [d]   cross-attention output projection */
  void *text_k, *text_v;       /* [B, T, d] keys / values of the instruction */
} wamc_layer_w;

/* Library version (WAMC_VERSION). */
int wamc_version(void);

/* Static text for a status code. */
const char* wamc_status_string(int status);

/* Detail of the last failing call on this thread ("" if none). */
const char* wamc_last_error(void);

/* Bytes of scratch workspace any call below needs for these sizes and a row
 * capacity of rows_cap rows per episode (the dense prefill uses rows_cap = N).
 * One workspace of this size serves every entry point.  For bf16 it includes
 * about 100 MiB for the kernels that split work across workgroups (partial
 * tiles and arrival counters); the calls clear what must start at zero, so
 * the workspace needs no initialisation.  Calls that share one workspace
 * must not overlap on the device (same stream, or synchronised). */
int wamc_workspace_bytes(const wamc_dims* dims, int32_t rows_cap, size_t* bytes);

/* Token scores (WAM-Cache §1, §4.2, §4.3).
 *   P_i = sum over layers l, heads h and action queries a of
 *         softmax_j(q_act[l,b,a,h] . K[l,b,j,h] / sqrt(dh))[i]
 *   U_i = sum_c (z[b,i,c] - zref[b,i,c])^2
 *   score_i = w_attn * P_i / (L*H*A) + w_surprise * U_i / sum_j U_j
 *   (the surprise term is 0 when sum_j U_j == 0).
 * z, zref: [B, N, d] act; q_act: [L, B, A, d] act; k_cache: [L, B, N, d] act,
 * the cache as it stands before this chunk's refresh.
 * mass_in (nullable, [B, N] f32): an attention mass supplied by a real action
 * expert; when given, q_act and k_cache may be NULL and P is not recomputed.
 * Outputs: score [B, N] f32; mass_out, surprise_out (nullable, [B, N] f32).
 * Bound by HBM: K is read twice (row max/sum pass, then mass pass). */
int wamc_score(const wamc_dims* dims, const void* z, const void* zref, const void* q_act,
               const void* k_cache, const float* mass_in, float* score, float* mass_out,
               float* surprise_out, void* ws, size_t ws_bytes, void* stream);

/* Refresh-set selection with the age bound (WAM-Cache §1, §4.4).
 *   forced = {i : age[b,i] >= G};  k_eff = min(max(k, |forced|), rows_cap)
 *   The refresh set is the k_eff tokens with the largest key
 *   (forced, score, -i): forced first, then higher score, then lower index;
 *   -0.0 ranks equal to +0.0 and NaN below every number.
 *   idx[b, 0..k_eff) = the set in ascending token order; idx[b, k_eff..N) = -1.
 *   age[b,i] <- 0 if refreshed else age[b,i] + 1.
 * score: [B, N] f32; age: [B, N] i32 in/out; k in [0, N]; rows_cap in [k, N]
 * (when more tokens are forced than rows_cap, the first rows_cap of them in
 * key order are refreshed and the rest stay due); idx: [B, N] i32 out;
 * k_eff: [B] i32 out; n_forced (nullable): [B] i32 out.
 * Bit-exact: a pure function of (score bits, ages, k, G, rows_cap). */
int wamc_select(const wamc_dims* dims, const float* score, int32_t* age, int32_t k,
                int32_t rows_cap, int32_t* idx, int32_t* k_eff, int32_t* n_forced, void* stream);

/* Gather the refreshed rows and store their reference embedding
 * (WAM-Cache §4.1: the reference embedding is the input embedding at the
 * token's most recent refresh):
 *   x[b, r, :] = float(z[b, idx[b,r], :]);  zref[b, idx[b,r], :] = z[b, idx[b,r], :]
 * for r < k_eff[b].  z, zref: [B, N, d] act; idx: [B, N] i32; k_eff: [B] i32;
 * x: [B, rows_cap, d] f32 out. */
int wamc_gather(const wamc_dims* dims, const void* z, void* zref, const int32_t* idx,
                const int32_t* k_eff, int32_t rows_cap, float* x, void* stream);

/* One DiT layer on the refreshed rows (WAM-Cache §3, §4.4):
 *   H1 = LN(x)*(1+scale1)+shift1;  [Q|Kn|Vn] = H1 W_qkv^T + b_qkv;
 *   K[idx[r]] <- Kn[r], V[idx[r]] <- Vn[r]   (before attention);
 *   O = per-head softmax(Q K^T / sqrt(dh)) V over all N cache rows;
 *   x += gate1 * (O W_o^T + b_o);
 *   with text (dims.n_text = T > 0): Qc = LN(x) W_qc^T + b_qc,
 *   x += softmax(Qc K_t^T / sqrt(dh)) V_t W_oc^T + b_oc over the T text keys;
 *   x += gate2 * (GELU(H2 W_1^T + b_1) W_2^T + b_2),  H2 = LN(x)*(1+scale2)+shift2
 * LN: no affine, biased variance, eps = dims.ln_eps; GELU: erf form.
 * layer: in [0, L) (bookkeeping only: w and the cache pointers are this layer's).
 * x: [B, rows_cap, d] f32 in/out (row r of episode b = token idx[b,r]).
 * idx (nullable = identity, rows are tokens 0..rows_cap-1): [B, N] i32.
 * k_eff (nullable = rows_cap rows in every episode): [B] i32.
 * k_cache_l, v_cache_l: [B, N, d] act, this layer's cache, updated in place.
 * bf16: H1, Q, K/V, O, H2 and the GELU output are rounded to bf16 (nearest
 * even); all accumulation and the residual stream are f32. */
int wamc_refresh_layer(const wamc_dims* dims, int32_t layer, const wamc_layer_w* w, float* x,
                       const int32_t* idx, const int32_t* k_eff, int32_t rows_cap,
                       void* k_cache_l, void* v_cache_l, void* ws, size_t ws_bytes, void* stream);

/* One whole refresh chunk (WAM-Cache §4.1-§4.4): wamc_score, then
 * wamc_select (or the given set), wamc_gather, then wamc_refresh_layer for
 * l = 0..L-1 with each layer's input the previous layer's output rows.
 * layers: HOST array of L wamc_layer_w.  z: [B,N,d] act (this chunk's tokens);
 * zref: [B,N,d] act in/out; q_act: [L,B,A,d] act; mass_in: nullable [B,N] f32;
 * k_cache, v_cache: [L,B,N,d] act in/out; age: [B,N] i32 in/out; k: requested
 * refresh count.
 * idx_override (nullable, [B,N] i32, ascending unique tokens) with
 * k_eff_override ([B] i32, required with it): use this refresh set instead of
 * scoring/selection; ages are then updated from it (score_out untouched).
 * Outputs: idx_out [B,N] i32 and k_eff_out [B] i32 (required); score_out
 * (nullable) [B,N] f32; layer_out (nullable) [L,B,rows_cap,d] f32: every
 * layer's output rows in idx order.
 * rows_cap (<= N) bounds k_eff.  When the library selects it must be at
 * least max(k, N - k), and N when G = 0 (WAMC_ERR_ARG otherwise): a token
 * forced at this chunk was not refreshed in the previous one, which
 * refreshed at least k tokens, so with ages that came from this library's
 * chunks at this k (or from a dense prefill) at most N - k tokens are forced
 * and the refresh set always fits, keeping every age <= G.  Ages supplied
 * from elsewhere can force more; the set is then cut to rows_cap by rank and
 * the forced tokens left out keep aging past G (wamc_select reports the
 * forced count).  With idx_override, rows_cap must hold the given set. */
int wamc_prefill_chunk(const wamc_dims* dims, const wamc_layer_w* layers, const void* z, void* zref,
                       const void* q_act, const float* mass_in, void* k_cache, void* v_cache,
                       int32_t* age, int32_t k, const int32_t* idx_override,
                       const int32_t* k_eff_override, int32_t* idx_out, int32_t* k_eff_out,
                       float* score_out, float* layer_out, int32_t rows_cap, void* ws,
                       size_t ws_bytes, void* stream);

/* The pages' own refresh rule, the union of two budgeted rank selections
 * (WAM-Cache §1 and §4.3: the tokens the action expert attended to most in
 * the preceding chunk and the tokens whose input embedding moved most since
 * their last refresh; §4.4: plus every token whose age reached the bound;
 * §5.3: a token chosen by several parts counts once):
 *   refresh set = top n_attn tokens by mass  |  top n_surprise tokens by
 *                 surprise  |  {i : age_i >= G},  k_eff = its size (variable)
 * ranked as in wamc_select (larger first, equal values to the lower index,
 * NaN below every number, -0 == +0); idx ascending, rest -1; ages as in
 * wamc_select.  n_attn = ceil(b_a N), n_surprise = ceil(b_s N) for budget
 * fractions (b_a, b_s), each in [0, N].  mass, surprise: [B, N] f32 (the
 * per-token P and U of wamc_score).  The set can hold every token, so there
 * is no row cap here. */
int wamc_select_union(const wamc_dims* dims, const float* mass, const float* surprise, int32_t* age,
                      int32_t n_attn, int32_t n_surprise, int32_t* idx, int32_t* k_eff, int32_t* n_forced,
                      void* stream);

/* wamc_prefill_chunk with the union rule in place of the fixed-k selection:
 * P and U of this chunk (P from q_act, or mass_in when given), then
 * wamc_select_union, wamc_gather and every layer on the k_eff rows.
 * rows_cap must be N (the union can hold every token); the kernels size
 * their work from k_eff on the device, so the spare capacity costs no time.
 * Other arguments as in wamc_prefill_chunk. */
int wamc_prefill_chunk_union(const wamc_dims* dims, const wamc_layer_w* layers, const void* z, void* zref,
                             const void* q_act, const float* mass_in, void* k_cache, void* v_cache,
                             int32_t* age, int32_t n_attn, int32_t n_surprise, int32_t* idx_out,
                             int32_t* k_eff_out, float* layer_out, int32_t rows_cap, void* ws,
                             size_t ws_bytes, void* stream);

/* Text keys and values of every layer from the instruction embeddings
 * (WAM-Cache §3): layers[l].text_k / text_v <- text W_kvc^T + b_kvc (K then
 * V halves), rounded to act.  text: [B, T, d] act.  Call once per episode,
 * before the dense prefill; needs dims.n_text > 0 and every layer's w_kvc,
 * b_kvc, text_k, text_v.  ws as for rows_cap = T. */
int wamc_text_kv(const wamc_dims* dims, const wamc_layer_w* layers, const void* text, void* ws, size_t ws_bytes,
                 void* stream);

/* Dense prefill (WAM-Cache §4.1: the chunk at episode onset): every token
 * through every layer, K/V written for all N tokens, age <- 0, zref <- z.
 * Also the speedup baseline.  layer_out (nullable): [L,B,N,d] f32. */
int wamc_dense_prefill(const wamc_dims* dims, const wamc_layer_w* layers, const void* z, void* zref,
                       void* k_cache, void* v_cache, int32_t* age, float* layer_out, void* ws,
                       size_t ws_bytes, void* stream);

/* wamc_prefill_chunk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same chunk, with the workspace taken from a static scratch
 * array of WAMC_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends (its address is looked up once per device on
 * the first call).  Returns WAMC_ERR_WORKSPACE, with nothing enqueued, when
 * wamc_workspace_bytes(dims, rows_cap) exceeds that size (the 30-layer
 * d=1536 chunk at rows_cap = 2808 needs about 250 MiB; the d=3072 four-episode
 * chunk does not fit).  Calls no allocating routine.  Every call on one GPU
 * shares that GPU's array and leaves its contents behind; the kernels clear
 * what must start at zero, but calls that overlap on one GPU (other streams,
 * other threads) race on it and must be serialised by the caller.  Other
 * arguments, validation and errors as in wamc_prefill_chunk (whose name the
 * argument messages carry). */
#define WAMC_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int wamc_prefill_chunk_noalloc(const wamc_dims* dims, const wamc_layer_w* layers, const void* z, void* zref,
                               const void* q_act, const float* mass_in, void* k_cache, void* v_cache,
                               int32_t* age, int32_t k, const int32_t* idx_override,
                               const int32_t* k_eff_override, int32_t* idx_out, int32_t* k_eff_out,
                               float* score_out, float* layer_out, int32_t rows_cap, void* stream);

/* Optional per-kernel timing, off by default.  While on, every kernel launch
 * carries a pair of HIP events (hipExtLaunchKernel) that the runtime stamps
 * with that kernel's own start and end on the launch stream; a step made of
 * several small kernels (the age update from a caller-given set) is timed by
 * events recorded around it.  Enabling clears the registry.  A diagnostic for
 * eager calls: leave it off while a stream is being captured into a graph.
 * wamc_timing_count returns the number of kernel kinds seen; wamc_timing_get
 * synchronises the recorded events and returns, for kind i, its name, the
 * number of launches and the summed launch durations in milliseconds. */
int wamc_timing_enable(int on);
int wamc_timing_count(void);
int wamc_timing_get(int i, const char** name, int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* WAMC_H */
