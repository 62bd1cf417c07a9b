"""Pins of the oracle's DiT block (WAM-Cache §3: self-attention + MLP, each
with a residual; every query attends over all keys) and of its bf16 storage
rounding (WAM-Cache §5.1: the models run in bfloat16).

Pinned against: a scalar pure-Python float64 second formulation of the whole
block on tiny shapes; library routines (torch CPU layer_norm, gelu and
scaled_dot_product_attention in float64; torch's bfloat16 conversion);
closed forms (LayerNorm moments, N = 1 attention, identical keys); and
hand-derived bf16 bit patterns.  Planted mistakes in the oracle must fail
these pins.
"""
import json
import math
import os
import struct
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import wamc_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = O.Precision("fp32")     # fp32 workloads: float64 arithmetic
BF = O.Precision("bf16")


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_golden_bits():
    with open(os.path.join(GOLDEN, "bf16_rounding.json")) as f:
        pairs = json.load(f)["pairs"]
    src = np.array([int(a, 16) for a, _, _ in pairs], dtype=np.uint32).view(np.float32)
    want = np.array([int(b, 16) for _, b, _ in pairs], dtype=np.uint32)
    got = O.round_bf16(src).view(np.uint32)
    assert got.tolist() == want.tolist()


def test_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-30, 30, 100000).astype(np.float32),
                        rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf], dtype=np.float32)
    r = O.round_bf16(x)
    assert np.isnan(r[:2]).all() and r[2] == np.inf and r[3] == -np.inf


# ---------------------------------------------------------------- pieces

def test_layer_norm_closed_form_and_torch():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((7, 33)) * 3 + 1.5
    eps = 1e-6
    Y = O.layer_norm(X, eps)
    assert np.allclose(Y.mean(axis=1), 0, atol=1e-12)
    var = X.var(axis=1)
    assert np.allclose(Y.var(axis=1), var / (var + eps), rtol=1e-12)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(X), (33,), eps=eps).numpy()
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_gelu_against_math_erf_and_torch():
    xs = np.linspace(-8, 8, 1001)
    want = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs])
    assert np.allclose(O.gelu(xs), want, rtol=1e-14, atol=1e-15)
    ref = torch.nn.functional.gelu(torch.from_numpy(xs)).numpy()
    assert np.allclose(O.gelu(xs), ref, rtol=1e-13, atol=1e-15)


def test_attention_against_torch_sdpa():
    rng = np.random.default_rng(1)
    m, N, H, dh = 5, 11, 3, 8
    Q = rng.standard_normal((m, H * dh))
    K = rng.standard_normal((N, H * dh))
    V = rng.standard_normal((N, H * dh))
    got = O.attention(Q, K, V, H)
    q = torch.from_numpy(Q).view(m, H, dh).transpose(0, 1)
    k = torch.from_numpy(K).view(N, H, dh).transpose(0, 1)
    v = torch.from_numpy(V).view(N, H, dh).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(m, H * dh)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(2)
    Q = rng.standard_normal((4, 12))
    # N = 1: the softmax is 1, so every query returns that value row
    K1, V1 = rng.standard_normal((1, 12)), rng.standard_normal((1, 12))
    assert np.allclose(O.attention(Q, K1, V1, 3), np.repeat(V1, 4, axis=0), atol=1e-15)
    # identical keys: uniform weights, output = mean of V
    K = np.repeat(rng.standard_normal((1, 12)), 9, axis=0)
    V = rng.standard_normal((9, 12))
    assert np.allclose(O.attention(Q, K, V, 3), np.repeat(V.mean(axis=0, keepdims=True), 4, axis=0), atol=1e-14)


# ---------------------------------------------------------------- whole block

def _rand_weights(rng, d, F, std=0.3):
    mod = rng.standard_normal((6, d)) * std
    mod[2] += 1
    mod[5] += 1
    return SimpleNamespace(w_qkv=rng.standard_normal((3 * d, d)) * std, b_qkv=rng.standard_normal(3 * d) * std,
                           w_o=rng.standard_normal((d, d)) * std, b_o=rng.standard_normal(d) * std,
                           w_1=rng.standard_normal((F, d)) * std, b_1=rng.standard_normal(F) * std,
                           w_2=rng.standard_normal((d, F)) * std, b_2=rng.standard_normal(d) * std, mod=mod)


def _scalar_bf16(v):
    """bf16 RNE of one float via struct (a second formulation)."""
    (b,) = struct.unpack("<I", struct.pack("<f", v))
    lsb = (b >> 16) & 1
    b = ((b + 0x7FFF + lsb) >> 16) << 16
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def scalar_text_kv(E, w, rnd=lambda v: v):
    """Text keys/values of one layer as scalar loops."""
    d = len(E[0])
    kv = [[rnd(w.b_kvc[o] + sum(E[j][c] * w.w_kvc[o][c] for c in range(d))) for o in range(2 * d)]
          for j in range(len(E))]
    return [r[:d] for r in kv], [r[d:] for r in kv]


def scalar_block(X, I, w, Kc, Vc, H, eps, rnd=lambda v: v, text=None):
    """The block written as plain scalar loops (float64), rounding through
    `rnd` at the storage points; `text` = (K_t, V_t) adds the cross-attention
    between self-attention and MLP."""
    m, d = len(X), len(X[0])
    N = len(Kc)
    dh = d // H
    F = len(w.b_1)
    Kc = [list(r) for r in Kc]
    Vc = [list(r) for r in Vc]

    def ln_mod(row, shift, scale):
        mu = sum(row) / d
        var = sum((v - mu) ** 2 for v in row) / d
        return [rnd((row[c] - mu) / math.sqrt(var + eps) * (1 + scale[c]) + shift[c]) for c in range(d)]

    X = [list(r) for r in X]
    h1 = [ln_mod(X[r], w.mod[0], w.mod[1]) for r in range(m)]
    q = [[0.0] * d for _ in range(m)]
    for r in range(m):
        for o in range(3 * d):
            acc = w.b_qkv[o]
            for c in range(d):
                acc += h1[r][c] * w.w_qkv[o][c]
            acc = rnd(acc)
            if o < d:
                q[r][o] = acc
            elif o < 2 * d:
                Kc[I[r]][o - d] = acc
            else:
                Vc[I[r]][o - 2 * d] = acc
    out = [[0.0] * d for _ in range(m)]
    for r in range(m):
        for h in range(H):
            s = []
            for j in range(N):
                s.append(sum(q[r][h * dh + c] * Kc[j][h * dh + c] for c in range(dh)) / math.sqrt(dh))
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            tot = sum(e)
            for c in range(dh):
                out[r][h * dh + c] = rnd(sum(e[j] / tot * Vc[j][h * dh + c] for j in range(N)))
    for r in range(m):
        proj = [w.b_o[o] + sum(out[r][c] * w.w_o[o][c] for c in range(d)) for o in range(d)]
        X[r] = [X[r][o] + w.mod[2][o] * proj[o] for o in range(d)]
    if text is not None:
        Kt, Vt = text
        T = len(Kt)
        zero = [0.0] * d
        h3 = [ln_mod(X[r], zero, zero) for r in range(m)]
        qc = [[rnd(w.b_qc[o] + sum(h3[r][c] * w.w_qc[o][c] for c in range(d))) for o in range(d)] for r in range(m)]
        oc = [[0.0] * d for _ in range(m)]
        for r in range(m):
            for h in range(H):
                s = [sum(qc[r][h * dh + c] * Kt[j][h * dh + c] for c in range(dh)) / math.sqrt(dh) for j in range(T)]
                mx = max(s)
                e = [math.exp(v - mx) for v in s]
                tot = sum(e)
                for c in range(dh):
                    oc[r][h * dh + c] = rnd(sum(e[j] / tot * Vt[j][h * dh + c] for j in range(T)))
        for r in range(m):
            X[r] = [X[r][o] + w.b_oc[o] + sum(oc[r][c] * w.w_oc[o][c] for c in range(d)) for o in range(d)]
    h2 = [ln_mod(X[r], w.mod[3], w.mod[4]) for r in range(m)]
    for r in range(m):
        g = []
        for f in range(F):
            a = w.b_1[f] + sum(h2[r][c] * w.w_1[f][c] for c in range(d))
            g.append(rnd(0.5 * a * (1 + math.erf(a / math.sqrt(2)))))
        down = [w.b_2[o] + sum(g[f] * w.w_2[o][f] for f in range(F)) for o in range(d)]
        X[r] = [X[r][o] + w.mod[5][o] * down[o] for o in range(d)]
    return np.array(X), np.array(Kc), np.array(Vc)


@pytest.mark.parametrize("m,N,d,H,F", [(3, 7, 8, 2, 12), (1, 5, 16, 4, 20), (4, 8, 12, 3, 9)])
def test_block_against_scalar_formulation(m, N, d, H, F):
    rng = np.random.default_rng(m * 100 + N)
    w = _rand_weights(rng, d, F)
    X = rng.standard_normal((m, d))
    I = np.sort(rng.choice(N, size=m, replace=False))
    Kc, Vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    Ko, Vo = Kc.copy(), Vc.copy()
    got = O.block(X.copy(), I, w, Ko, Vo, H, 1e-6, F64)
    want, Kw, Vw = scalar_block(X, I, w, Kc, Vc, H, 1e-6)
    assert np.allclose(got, want, rtol=1e-11, atol=1e-11)
    assert np.allclose(Ko, Kw, rtol=1e-12, atol=1e-12)
    assert np.allclose(Vo, Vw, rtol=1e-12, atol=1e-12)
    untouched = np.setdiff1d(np.arange(N), I)
    assert np.array_equal(Ko[untouched], Kc[untouched])


def _text_weights(rng, w, d, std=0.3):
    w.w_qc, w.b_qc = rng.standard_normal((d, d)) * std, rng.standard_normal(d) * std
    w.w_kvc, w.b_kvc = rng.standard_normal((2 * d, d)) * std, rng.standard_normal(2 * d) * std
    w.w_oc, w.b_oc = rng.standard_normal((d, d)) * std, rng.standard_normal(d) * std
    return w


@pytest.mark.parametrize("m,N,T,d,H,F", [(3, 7, 1, 8, 2, 12), (2, 5, 3, 16, 4, 20), (4, 8, 5, 12, 3, 9)])
def test_block_with_text_against_scalar_formulation(m, N, T, d, H, F):
    """The text cross-attention (WAM-Cache §3: SA, CA, MLP, each with a
    residual) against the scalar loops, text keys/values included."""
    rng = np.random.default_rng(m * 1000 + N * 10 + T)
    w = _text_weights(rng, _rand_weights(rng, d, F), d)
    E = rng.standard_normal((T, d))
    X = rng.standard_normal((m, d))
    I = np.sort(rng.choice(N, size=m, replace=False))
    Kc, Vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    Kt, Vt = O.text_kv(E, w, F64)
    Kts, Vts = scalar_text_kv(E.tolist(), w)
    assert np.allclose(Kt, Kts, rtol=1e-12, atol=1e-12) and np.allclose(Vt, Vts, rtol=1e-12, atol=1e-12)
    Ko, Vo = Kc.copy(), Vc.copy()
    got = O.block(X.copy(), I, w, Ko, Vo, H, 1e-6, F64, text=(Kt, Vt))
    want, Kw, Vw = scalar_block(X, I, w, Kc, Vc, H, 1e-6, text=(Kts, Vts))
    assert np.allclose(got, want, rtol=1e-11, atol=1e-11)
    assert np.allclose(Ko, Kw, rtol=1e-12, atol=1e-12)


def test_text_cross_attention_special_cases():
    """A zero output projection leaves the block bitwise as without text; a
    single text token gives every row the same cross-attention output
    V_t W_oc^T + b_oc (its softmax weight is 1)."""
    rng = np.random.default_rng(3)
    m, N, d, H, F = 4, 9, 12, 3, 10
    w = _text_weights(rng, _rand_weights(rng, d, F), d)
    X = rng.standard_normal((m, d))
    I = np.array([0, 3, 4, 8])
    Kc, Vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    E = rng.standard_normal((3, d))
    w0 = SimpleNamespace(**vars(w))
    w0.w_oc, w0.b_oc = np.zeros((d, d)), np.zeros(d)
    a = O.block(X.copy(), I, w0, Kc.copy(), Vc.copy(), H, 1e-6, F64, text=O.text_kv(E, w0, F64))
    b = O.block(X.copy(), I, w0, Kc.copy(), Vc.copy(), H, 1e-6, F64)
    assert np.array_equal(a, b)
    # single token; MLP switched off (zero weights and biases) so the output
    # is the post-attention stream plus the cross-attention branch
    w1 = SimpleNamespace(**vars(w))
    w1.w_1, w1.b_1, w1.w_2, w1.b_2 = np.zeros_like(w.w_1), np.zeros_like(w.b_1), np.zeros_like(w.w_2), np.zeros_like(w.b_2)
    Kt, Vt = O.text_kv(E[:1], w1, F64)
    with_t = O.block(X.copy(), I, w1, Kc.copy(), Vc.copy(), H, 1e-6, F64, text=(Kt, Vt))
    without = O.block(X.copy(), I, w1, Kc.copy(), Vc.copy(), H, 1e-6, F64)
    branch = Vt[0] @ w1.w_oc.T + w1.b_oc
    assert np.allclose(with_t - without, np.repeat(branch[None], m, axis=0), rtol=1e-12, atol=1e-12)


def test_block_bf16_storage_points():
    """bf16 mode: rounding happens at the storage points only; compared with
    the scalar formulation rounding at the same points."""
    rng = np.random.default_rng(11)
    m, N, d, H, F = 3, 6, 8, 2, 10
    w64 = _rand_weights(rng, d, F)
    w = SimpleNamespace(**{k: O.round_bf16(np.asarray(v, dtype=np.float32)) for k, v in vars(w64).items()})
    X = rng.standard_normal((m, d)).astype(np.float32)
    I = np.array([0, 2, 5])
    Kc = O.round_bf16(rng.standard_normal((N, d)).astype(np.float32))
    Vc = O.round_bf16(rng.standard_normal((N, d)).astype(np.float32))
    Ko, Vo = Kc.copy(), Vc.copy()
    got = O.block(X.copy(), I, w, Ko, Vo, H, 1e-6, BF)
    assert np.array_equal(O.round_bf16(Ko), Ko) and np.array_equal(O.round_bf16(Vo), Vo)
    wd = SimpleNamespace(**{k: np.asarray(v, dtype=np.float64) for k, v in vars(w).items()})
    want, Kw, Vw = scalar_block(X.astype(np.float64), I, wd, Kc.astype(np.float64), Vc.astype(np.float64),
                                H, 1e-6, rnd=_scalar_bf16)
    # float32 vs float64 accumulation may flip an occasional bf16 rounding
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 1e-2
    assert np.abs(Ko - Kw).max() <= 2 ** -6 * np.abs(Kw).max()


# ---------------------------------------------------------------- planted mistakes

def _pin_block():
    test_block_against_scalar_formulation(3, 7, 8, 2, 12)


def test_planted_gelu_tanh_is_caught(monkeypatch):
    def tanh_gelu(x):
        return 0.5 * x * (1 + np.tanh(np.sqrt(2 / np.pi) * (x + 0.044715 * x ** 3)))
    monkeypatch.setattr(O, "gelu", tanh_gelu)
    with pytest.raises(AssertionError):
        _pin_block()


def test_planted_unbiased_variance_is_caught(monkeypatch):
    def wrong_ln(X, eps):
        mu = X.mean(axis=1, keepdims=True)
        return (X - mu) / np.sqrt(X.var(axis=1, ddof=1, keepdims=True) + eps)
    monkeypatch.setattr(O, "layer_norm", wrong_ln)
    with pytest.raises(AssertionError):
        _pin_block()


def test_planted_missing_scale_is_caught(monkeypatch):
    def no_scale(Q, Kc, Vc, n_heads):
        m, d = Q.shape
        dh = d // n_heads
        out = np.empty_like(Q)
        for h in range(n_heads):
            c = slice(h * dh, (h + 1) * dh)
            out[:, c] = O.softmax_rows(Q[:, c] @ Kc[:, c].T) @ Vc[:, c]
        return out
    monkeypatch.setattr(O, "attention", no_scale)
    with pytest.raises(AssertionError):
        _pin_block()


def test_planted_transposed_heads_are_caught(monkeypatch):
    real = O.attention

    def swapped(Q, Kc, Vc, n_heads):   # keys of the wrong head
        return real(Q, np.roll(Kc, Kc.shape[1] // n_heads, axis=1), Vc, n_heads)
    monkeypatch.setattr(O, "attention", swapped)
    with pytest.raises(AssertionError):
        _pin_block()
