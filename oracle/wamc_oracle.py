"""CPU oracle of the staleness-bounded sparse KV-refresh prefill (WAM-Cache).

TEST INFRASTRUCTURE ONLY.  This module is imported by the test-suite, by the
smoke check of the graft entry point and by the CPU-baseline leg of the
benchmark -- never by the product path, which must fail loudly when its HIP
library is missing.  It shares no code with the HIP path: plain numpy (scipy
only for erf), one step after another, in the order the method states them.

What it computes, with the page each step follows (titles as printed):

* "WAM-Cache: Staleness-Bounded KV Reuse for Efficient World Action Models"
  - §3 "Preliminaries": a DiT module is self-attention + MLP, each with a
    residual; Q/K/V are linear projections of the module input; every query
    attends over all S_v keys and values; the module's text cross-attention
    (keys and values projected from the instruction) is optional here.
  - §4.1 "Overview": per-token state = layerwise cached K/V, a reference
    embedding stored at the token's last refresh, an age counter of
    consecutive reuses and the action expert's attention mass from the
    preceding chunk; chunk 0 is a dense prefill with all ages zero.
  - §1 "Introduction" and §4.2-4.4: refresh-set signals -- latent surprise
    (how far the input embedding moved since the last refresh), action
    attention mass, and an age bound that forces a refresh after a fixed
    number of consecutive reuses; the prefill then runs only on the refresh
    set while refreshed queries attend over fresh and retained K/V.
  - §5.2 "CUDA latency": prefill cost scales with the recompute ratio, so the
    speedup is bounded by its inverse.
* "RealtimeWAM" App. D.3 "Recursive reuse": an age cap of two permits at most
  two consecutive reuses (fixes the age semantics below).

Readings where the pages are silent or garbled (the display equations of
WAM-Cache §4.2-4.4 are lost in the text):

* one combined score = w_a * P_i / (L*H*A) + w_s * U_i / sum(U), with a fixed
  requested count k (the default rule);
* the page's own rule, the union of two budgeted rank selections (§1, §4.3,
  §5.3): the ceil(b_a*N) tokens of largest attention mass, the ceil(b_s*N)
  tokens of largest surprise, and the forced tokens, each token counted once
  (`select_union`);
* P_i = sum over layers, heads and action queries of the row-softmax
  probability of token i, computed from the supplied queries against the
  cache as it stands before this chunk's refresh;
* U_i = squared L2 distance of z_t[i] from the reference embedding stored at
  token i's last refresh;
* forced iff age >= G; forced tokens count toward k and
  k_eff = max(k, #forced); ranking key (forced, score, -index) descending,
  -0.0 == +0.0, NaN below every number; the refresh set is kept in
  ascending token order; refreshed -> age 0, otherwise age + 1;
* one refresh set shared by all layers; a refreshed row's layer-l input is its
  own layer-(l-1) output of this chunk;
* block: LayerNorm (eps, biased variance, no affine), modulation
  LN*(1+scale)+shift, QKV with bias, the fresh K/V are written into the cache
  *before* attention, softmax(Q K^T / sqrt(dh)) V over all N cached keys,
  gated residual out-projection, a second modulated LN, GELU (erf form) MLP
  with a gated residual;
* optional text cross-attention between the two (§3: SA, CA, MLP): queries
  from an unmodulated LN of the rows with bias, keys/values projected from
  the instruction's embeddings once per episode, per-head softmax over the T
  text tokens, ungated residual out-projection;
* precision: fp32 workloads run here in float64 with no rounding; bf16
  workloads run in float32 arithmetic with round-to-nearest-even bf16 at the
  storage points (weights, z, zref, Qa, H1, Q, K/V cache, attention output,
  H2, GELU output), the residual stream staying float32.

Parity pins: every function below is checked by the CPU tests against closed
forms, library routines, brute force, hand-worked values or a scalar second
formulation (surprise, combine and the reference update against hand-worked
multi-chunk values), except full multi-chunk rollouts with stale caches
("parity unpinned" beyond the invariants the tests check: they have no
printed worked example).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf


# --------------------------------------------------------------------------
# precision handling
# --------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even; returns float32.

    bfloat16 keeps the top 16 bits of an IEEE binary32 word.  Adding
    0x7FFF plus the lowest kept bit and truncating is round-half-to-even.
    NaN stays NaN (quiet bit forced so truncation cannot make it inf).
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    bits = x32.view(np.uint32)
    # no wrap-around in 32 bits: the largest non-NaN pattern is 0xFF800000
    r = bits + (np.uint32(0x7FFF) + ((bits >> 16) & np.uint32(1)))
    r &= np.uint32(0xFFFF0000)
    nan = np.isnan(x32)
    if nan.any():
        r = np.where(nan, (bits | np.uint32(0x00400000)) & np.uint32(0xFFFF0000), r)
    return r.view(np.float32).reshape(x32.shape)


class Precision:
    """fp32 workloads -> float64 arithmetic, no rounding.
    bf16 workloads -> float32 arithmetic, bf16 rounding at storage points."""

    def __init__(self, dtype: str):
        if dtype not in ("fp32", "bf16"):
            raise ValueError(dtype)
        self.dtype = dtype
        self.bf16 = dtype == "bf16"
        self.acc = np.float32 if self.bf16 else np.float64

    def load(self, x) -> np.ndarray:
        """A stored input, as an array of the arithmetic type."""
        return np.asarray(x).astype(self.acc)

    def store(self, x: np.ndarray) -> np.ndarray:
        """Value written to a storage point (cache, Q, H1, O, H2, GELU out)."""
        if self.bf16:
            return round_bf16(x)
        return np.asarray(x, dtype=self.acc)


# --------------------------------------------------------------------------
# the DiT block (WAM-Cache §3; refresh variant §4.1/§4.4)
# --------------------------------------------------------------------------

def layer_norm(X: np.ndarray, eps: float) -> np.ndarray:
    """Row LayerNorm without affine parameters: (x - mean) / sqrt(var + eps),
    var the biased (population) variance."""
    mu = X.mean(axis=1, keepdims=True)
    var = ((X - mu) ** 2).mean(axis=1, keepdims=True)
    return (X - mu) / np.sqrt(var + eps)


def gelu(x: np.ndarray) -> np.ndarray:
    """GELU(x) = x/2 * (1 + erf(x / sqrt(2)))."""
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0).astype(x.dtype)))


def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted first."""
    E = S - S.max(axis=1, keepdims=True)
    np.exp(E, out=E)
    E /= E.sum(axis=1, keepdims=True)
    return E


def attention(Q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, n_heads: int) -> np.ndarray:
    """Multi-head attention of the m query rows over all N cache rows, per
    head softmax(Q_h K_h^T / sqrt(dh)) V_h.  No mask."""
    m, d = Q.shape
    dh = d // n_heads
    O = np.empty((m, d), dtype=Q.dtype)
    scale = Q.dtype.type(1.0 / math.sqrt(dh))
    for h in range(n_heads):
        cols = slice(h * dh, (h + 1) * dh)
        P = softmax_rows((Q[:, cols] @ Kc[:, cols].T) * scale)
        O[:, cols] = P @ Vc[:, cols]
    return O


def text_kv(E: np.ndarray, w, prec: Precision):
    """Keys and values of the text cross-attention of one layer (WAM-Cache §3:
    the cross-attention layer attends to keys and values projected from the
    text embeddings): [K_t | V_t] = E W_kvc^T + b_kvc, rows of W_kvc K then
    V.  They depend on the instruction only, so they are computed once per
    episode and kept."""
    d = E.shape[1]
    ld = prec.load
    KV = ld(E) @ ld(w.w_kvc).T + ld(w.b_kvc)
    return prec.store(KV[:, :d]), prec.store(KV[:, d:])


def block(X: np.ndarray, I: np.ndarray, w, Kc: np.ndarray, Vc: np.ndarray,
          n_heads: int, eps: float, prec: Precision, text=None) -> np.ndarray:
    """One DiT layer applied to the rows X (token ids I, ascending).

    Kc, Vc are this layer's cache [N, d]; rows I are overwritten with the
    fresh keys/values before attention, so refreshed queries see their own
    fresh keys and every other token's retained ones.  With `text` = (K_t,
    V_t) the module also runs its text cross-attention between self-attention
    and the MLP (WAM-Cache §3: SA, CA, MLP, each with a residual): the
    queries come from an unmodulated LayerNorm of the rows, the residual is
    ungated.  Returns the layer's output rows (the residual stream,
    arithmetic precision).
    """
    d = X.shape[1]
    ld = prec.load
    mod = ld(w.mod)
    shift1, scale1, gate1, shift2, scale2, gate2 = mod
    H1 = prec.store(layer_norm(X, eps) * (1 + scale1) + shift1)
    QKV = H1 @ ld(w.w_qkv).T + ld(w.b_qkv)
    Q = prec.store(QKV[:, :d])
    Kc[I] = prec.store(QKV[:, d:2 * d])
    Vc[I] = prec.store(QKV[:, 2 * d:])
    O = prec.store(attention(Q, Kc, Vc, n_heads))
    X = X + gate1 * (O @ ld(w.w_o).T + ld(w.b_o))
    if text is not None:
        Kt, Vt = text
        H3 = prec.store(layer_norm(X, eps))
        Qc = prec.store(H3 @ ld(w.w_qc).T + ld(w.b_qc))
        Oc = prec.store(attention(Qc, Kt, Vt, n_heads))
        X = X + (Oc @ ld(w.w_oc).T + ld(w.b_oc))
    H2 = prec.store(layer_norm(X, eps) * (1 + scale2) + shift2)
    G = prec.store(gelu(H2 @ ld(w.w_1).T + ld(w.b_1)))
    X = X + gate2 * (G @ ld(w.w_2).T + ld(w.b_2))
    return X


# --------------------------------------------------------------------------
# per-token state and the dense prefill (WAM-Cache §4.1)
# --------------------------------------------------------------------------

@dataclass
class State:
    """Per-episode cache state: K, V [L, N, d]; age [N] int; zref [N, d];
    text: per layer (K_t, V_t) of the instruction, or None (no text
    cross-attention)."""
    K: np.ndarray
    V: np.ndarray
    age: np.ndarray
    zref: np.ndarray
    text: Optional[list] = None

    def copy(self) -> "State":
        return State(self.K.copy(), self.V.copy(), self.age.copy(), self.zref.copy(), self.text)


def dense_prefill(z: np.ndarray, weights: Sequence, n_heads: int, eps: float,
                  prec: Precision, text_emb: Optional[np.ndarray] = None):
    """Chunk 0: every token through every layer; ages 0 and zref = z.  With
    text embeddings E [T, d] every layer also runs its text cross-attention
    (its text keys/values, computed here, are kept in the state).

    Returns (state, [X_l for each layer])."""
    N, d = z.shape
    L = len(weights)
    K = np.zeros((L, N, d), dtype=prec.acc)
    V = np.zeros((L, N, d), dtype=prec.acc)
    text = None if text_emb is None else [text_kv(text_emb, weights[l], prec) for l in range(L)]
    X = prec.load(z)
    I = np.arange(N)
    outs = []
    for l in range(L):
        X = block(X, I, weights[l], K[l], V[l], n_heads, eps, prec, None if text is None else text[l])
        outs.append(X.copy())
    return State(K, V, np.zeros(N, dtype=np.int64), prec.load(z).copy(), text), outs


# --------------------------------------------------------------------------
# scoring (WAM-Cache §1, §4.2, §4.3)
# --------------------------------------------------------------------------

def attention_mass(qa: np.ndarray, K: np.ndarray, n_heads: int, prec: Precision) -> np.ndarray:
    """P_i = sum over layers l, heads h and action queries a of
    softmax_j(qa[l,a,h] . K[l,j,h] / sqrt(dh))[i]."""
    L, N, d = K.shape
    dh = d // n_heads
    scale = prec.acc(1.0 / math.sqrt(dh))
    P = np.zeros(N, dtype=prec.acc)
    for l in range(L):
        q = prec.load(qa[l])
        for h in range(n_heads):
            cols = slice(h * dh, (h + 1) * dh)
            probs = softmax_rows((q[:, cols] @ K[l][:, cols].T) * scale)
            P += probs.sum(axis=0)
    return P


def surprise(z: np.ndarray, zref: np.ndarray, prec: Precision) -> np.ndarray:
    """U_i = sum_c (z[i,c] - zref[i,c])^2: the squared Euclidean distance
    over the d channels between token i's current input embedding and its
    reference embedding (WAM-Cache §4.2 "Latent Surprise": how far the
    embedding moved since the token was last refreshed; §4.1 for the
    reference)."""
    diff = prec.load(z) - prec.load(zref)
    return (diff * diff).sum(axis=1)


def combine(P: np.ndarray, U: np.ndarray, n_layers: int, n_heads: int, n_action: int,
            w_attn: float, w_surprise: float) -> np.ndarray:
    """score_i = w_a * P_i/(L*H*A) + w_s * U_i/sum(U) (the second term is 0
    when nothing moved).  Returned as float32, the format selection uses."""
    total = U.sum()
    s = w_attn * (P / (n_layers * n_heads * n_action))
    if total > 0:
        s = s + w_surprise * (U / total)
    return np.asarray(s, dtype=np.float32)


def score(z, zref, qa, K, n_heads: int, w_attn: float, w_surprise: float,
          prec: Precision, mass: Optional[np.ndarray] = None, n_action: Optional[int] = None):
    """Returns (score float32 [N], P, U).  `mass` replaces P when an action
    expert supplies its own attention mass: it is the same sum over layers,
    heads and action queries, so it is normalised by the same L*H*A
    (`n_action` = A must then be given)."""
    L = K.shape[0]
    if mass is None:
        A = qa.shape[1]
        P = attention_mass(qa, K, n_heads, prec)
    else:
        if n_action is None:
            raise ValueError("a supplied attention mass needs n_action")
        A = n_action
        P = prec.load(mass)
    U = surprise(z, zref, prec)
    return combine(P, U, L, n_heads, A, w_attn, w_surprise), P, U


# --------------------------------------------------------------------------
# selection with the age bound (WAM-Cache §1, §4.4; RealtimeWAM App. D.3)
# --------------------------------------------------------------------------

def rank_key(forced: bool, s: float, i: int):
    """Total order used for selection: forced first, then larger score, then
    lower index.  NaN ranks below every number; -0.0 equals +0.0."""
    isnum = not math.isnan(s)
    return (forced, isnum, (s + 0.0) if isnum else 0.0, -i)


def select(score_f32: np.ndarray, age: np.ndarray, k: int, G: int,
           cap: Optional[int] = None):
    """Refresh-set selection.

    forced = {i : age_i >= G}; k_eff = max(k, #forced) (capped by `cap`, the
    row capacity, when given); the refresh set is the k_eff largest keys of
    rank_key; returned in ascending token order with the updated ages
    (0 if refreshed, else +1).  Returns (idx int32, k_eff, new_age, n_forced).
    """
    N = len(score_f32)
    if not (0 <= k <= N):
        raise ValueError("k out of range")
    forced = np.asarray(age) >= G
    n_forced = int(forced.sum())
    k_eff = max(k, n_forced)
    if cap is not None:
        k_eff = min(k_eff, cap)
    keys = [rank_key(bool(forced[i]), float(score_f32[i]), i) for i in range(N)]
    order = sorted(range(N), key=lambda i: keys[i], reverse=True)
    idx = np.array(sorted(order[:k_eff]), dtype=np.int32)
    return idx, k_eff, ages_after(age, idx), n_forced


def budget_count(b: float, N: int) -> int:
    """ceil(b * N) computed exactly for a budget given as a decimal fraction
    (0.4 * 4680 is 1872, not 1873 as float rounding would give)."""
    from fractions import Fraction
    if b < 0:
        raise ValueError("budget must be >= 0")
    return min(N, math.ceil(Fraction(repr(float(b))) * N))


def top_by(values_f32: np.ndarray, n: int) -> np.ndarray:
    """The n tokens with the largest value, ascending: larger value first,
    equal values -> lower index first, NaN below every number, -0.0 == +0.0."""
    N = len(values_f32)
    n = max(0, min(n, N))
    keys = [rank_key(False, float(values_f32[i]), i) for i in range(N)]
    order = sorted(range(N), key=lambda i: keys[i], reverse=True)
    return np.array(sorted(order[:n]), dtype=np.int32)


def select_union(mass_f32: np.ndarray, surprise_f32: np.ndarray, age: np.ndarray, n_attn: int,
                 n_surprise: int, G: int):
    """The page's refresh rule (WAM-Cache §1 and §4.3: union of the
    action-attention set and the latent-surprise set; §4.4: plus every token
    whose age reached the bound; §5.3: tokens chosen by both signals are
    counted once).  P_t = top n_attn tokens by attention mass, S_t = top
    n_surprise by surprise, F_t = {age >= G}; the refresh set is
    P_t | S_t | F_t in ascending token order, k_eff = its size (variable);
    ages 0 on the set, +1 elsewhere.  Returns (idx, k_eff, new_age, n_forced)."""
    N = len(mass_f32)
    forced = np.flatnonzero(np.asarray(age) >= G)
    R = set(top_by(mass_f32, n_attn).tolist()) | set(top_by(surprise_f32, n_surprise).tolist())
    R |= set(forced.tolist())
    idx = np.array(sorted(R), dtype=np.int32)
    assert len(idx) <= N
    return idx, len(idx), ages_after(age, idx), int(len(forced))


def ages_after(age: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Age update for a refresh set: refreshed tokens restart at 0, all others
    have been reused one more chunk."""
    new = np.asarray(age, dtype=np.int64) + 1
    new[np.asarray(idx, dtype=np.int64)] = 0
    return new


def update_reference(zref: np.ndarray, z: np.ndarray, idx: np.ndarray) -> None:
    """The reference embedding of a token is the input embedding it had at
    its most recent refresh (WAM-Cache §4.1): refreshed rows take this
    chunk's z, every other row keeps the one stored when it was last
    refreshed (so a token that moves while being reused accumulates
    surprise against that older embedding)."""
    zref[idx] = z[idx]


# --------------------------------------------------------------------------
# one refresh chunk (WAM-Cache §4.1-4.4)
# --------------------------------------------------------------------------

@dataclass
class ChunkResult:
    score: np.ndarray
    mass: np.ndarray
    surprise: np.ndarray
    idx: np.ndarray
    k_eff: int
    n_forced: int
    outs: List[np.ndarray] = field(default_factory=list)   # X_l rows, idx order


def refresh_chunk(state: State, z: np.ndarray, qa: Optional[np.ndarray], weights: Sequence,
                  k: int, G: int, n_heads: int, eps: float, w_attn: float, w_surprise: float,
                  prec: Precision, idx_override: Optional[np.ndarray] = None,
                  mass: Optional[np.ndarray] = None, cap: Optional[int] = None,
                  union: Optional[tuple] = None) -> ChunkResult:
    """Score against the current cache, select, gather the refreshed rows
    (and store their reference embedding), then run every layer on them.
    `union` = (n_attn, n_surprise) selects with the union rule instead of the
    fixed-k combined score (k is then ignored).  `state` is updated in place."""
    s, P, U = score(z, state.zref, qa, state.K, n_heads, w_attn, w_surprise, prec, mass,
                    n_action=None if qa is None else qa.shape[1])
    if idx_override is None and union is not None:
        idx, k_eff, age, n_forced = select_union(np.asarray(P, dtype=np.float32), np.asarray(U, dtype=np.float32),
                                                 state.age, union[0], union[1], G)
    elif idx_override is None:
        idx, k_eff, age, n_forced = select(s, state.age, k, G, cap)
    else:
        idx = np.array(sorted(set(int(i) for i in idx_override)), dtype=np.int32)
        k_eff, n_forced = len(idx), int((np.asarray(state.age) >= G).sum())
        age = ages_after(state.age, idx)
    state.age = age
    zl = prec.load(z)
    X = zl[idx].copy()
    update_reference(state.zref, zl, idx)
    outs = []
    for l in range(len(weights)):
        X = block(X, idx, weights[l], state.K[l], state.V[l], n_heads, eps, prec,
                  None if state.text is None else state.text[l])
        outs.append(X.copy())
    return ChunkResult(s, P, U, idx, k_eff, n_forced, outs)


# --------------------------------------------------------------------------
# cost model (WAM-Cache §5.2 "CUDA latency", §5.3)
# --------------------------------------------------------------------------

def prefill_flops(rows: int, n_tokens: int, n_layers: int, d: int, d_ffn: int) -> int:
    """Multiply-add FLOPs of the prefill on `rows` rows: per row and layer
    QKV 6d^2, out-projection 2d^2, attention over all N keys 4Nd, MLP 4dF."""
    per_row = 8 * d * d + 4 * n_tokens * d + 4 * d * d_ffn
    return rows * n_layers * per_row
