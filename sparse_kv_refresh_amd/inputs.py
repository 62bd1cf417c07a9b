"""Seeded synthetic inputs for the staleness-bounded sparse KV-refresh prefill.

This module only *draws* inputs: DiT-shaped weights, observation latents with a
static background and moving regions, the patch embedding that turns a latent
into visual tokens, action-expert query stand-ins and initial cache ages.  It
holds none of the method's arithmetic (no scoring, selection, normalisation,
attention or MLP) and imports nothing from the oracle or from the HIP path, so
both sides can be fed the same bytes.

Why these shapes: WAM-Cache (paperpeel 2610.11401, §1) observes that from one
chunk to the next, motion in a manipulation scene is mostly confined to the
end-effector and the target object; the latents below are a static scene plus
one drifting patch or a few moving blobs.  §3 of the same page defines the
visual tokens z_t as a patch-embedding projection of the observation latent;
here that projection is a seeded linear map from 16 latent channels to d.

bf16 workloads: every stored input is rounded once, round-to-nearest-even, to
a bf16-representable float32 value, so the CPU oracle and the GPU library see
identical bits (the GPU side converts the float32 array to bfloat16 exactly).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

LATENT_CH = 16

SEED_WEIGHTS = 0
SEED_PATCH = 1
SEED_LATENT = 100
SEED_QUERY = 200
SEED_AGES = 300
SEED_TEXT = 400
SEED_TEXT_WEIGHTS = 7


@dataclass(frozen=True)
class Workload:
    """Shapes and knobs of one synthetic workload."""
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    d_ffn: int
    views: int
    rows: int
    cols: int
    n_action: int
    k: int
    age_bound: int
    dtype: str                   # "fp32" or "bf16"
    batch: int = 1
    chunks: int = 8              # chunk 0 is the dense prefill
    latent: str = "blob"         # "blob", "patch", "stack", "episodes"
    w_attn: float = 0.4
    w_surprise: float = 0.1
    ln_eps: float = 1e-6
    random_initial_ages: bool = False   # ages ~ U{0..G} after the dense chunk
    n_text: int = 0                     # instruction tokens of the text cross-attention (0: none)

    @property
    def n_tokens(self) -> int:
        return self.views * self.rows * self.cols

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Named presets.  c1..c5 follow the five workloads of the synthetic benchmark
# plan; t_* are reduced shapes that still span several GEMM/attention tiles
# with ragged tails, sized so the CPU oracle finishes in seconds.
PRESETS: Dict[str, Workload] = {
    # 2-layer fp32 DiT, d=128, 4 heads, FFN 512; 16x16 grid; moving 4x4 blob.
    "c1_tiny": Workload("c1_tiny", 2, 128, 4, 512, 1, 16, 16, 32, 64, 4, "fp32",
                        chunks=8, latent="blob"),
    # single bf16 layer, d=1536, 12 heads, FFN 8960; 64x64 grid, k = 60 % of N.
    "c2_layer": Workload("c2_layer", 1, 1536, 12, 8960, 1, 64, 64, 64, 2458, 3, "bf16",
                         chunks=2, latent="patch", random_initial_ages=True),
    # 30-layer bf16 stack, 3 views x 30x52 = 4680 tokens, k = 60 %.
    "c3_stack": Workload("c3_stack", 30, 1536, 12, 8960, 3, 30, 52, 64, 2808, 3, "bf16",
                         chunks=16, latent="stack"),
    # the 30-layer stack with the module's text cross-attention over 128
    # instruction tokens
    "c3_text": Workload("c3_text", 30, 1536, 12, 8960, 3, 30, 52, 64, 2808, 3, "bf16",
                        chunks=16, latent="stack", n_text=128),
    # the 30-layer stack at the small context of the latency experiment: one
    # view of 36x30 = 1080 tokens, k = 631 (the 0.584 refresh ratio), G = 2
    "c3_ctx1080": Workload("c3_ctx1080", 30, 1536, 12, 8960, 1, 36, 30, 64, 631, 2, "bf16",
                           chunks=16, latent="stack"),
    # 20-layer d=3072 bf16, 2 views x 64x64 = 8192 tokens, 4 episodes, k = 50 %.
    "c5_large": Workload("c5_large", 20, 3072, 24, 12288, 2, 64, 64, 128, 4096, 4, "bf16",
                         batch=4, chunks=8, latent="episodes"),
    # reduced shapes for parity tests
    "t_fp32_ragged": Workload("t_fp32_ragged", 2, 96, 3, 200, 1, 13, 23, 19, 101, 2, "fp32",
                              chunks=4, latent="blob"),
    "t_bf16_small": Workload("t_bf16_small", 2, 256, 2, 640, 1, 20, 35, 40, 300, 2, "bf16",
                             chunks=4, latent="blob"),
    "t_bf16_batch": Workload("t_bf16_batch", 2, 256, 2, 512, 2, 17, 19, 64, 330, 3, "bf16",
                             batch=3, chunks=4, latent="episodes"),
    "t_bf16_stack": Workload("t_bf16_stack", 4, 1536, 12, 8960, 3, 30, 52, 64, 2808, 3, "bf16",
                             chunks=3, latent="stack"),
    # with the text cross-attention: 77 instruction tokens (ragged against
    # the 64-key tiles)
    "t_bf16_text": Workload("t_bf16_text", 2, 256, 2, 640, 1, 20, 35, 40, 300, 2, "bf16",
                            chunks=4, latent="blob", n_text=77),
    "t_fp32_text": Workload("t_fp32_text", 2, 128, 4, 512, 1, 16, 16, 32, 64, 4, "fp32",
                            chunks=4, latent="blob", n_text=23),
}


def preset(name: str, **overrides) -> Workload:
    wl = PRESETS[name]
    return wl.with_(**overrides) if overrides else wl


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even).

    Storage-format conversion of generated inputs; NaN/inf never occur here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _store(wl: Workload, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return to_bf16_values(x) if wl.dtype == "bf16" else x


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


@dataclass
class LayerWeights:
    w_qkv: np.ndarray   # [3d, d]  rows: Q, K, V
    b_qkv: np.ndarray   # [3d]
    w_o: np.ndarray     # [d, d]
    b_o: np.ndarray     # [d]
    w_1: np.ndarray     # [F, d]
    b_1: np.ndarray     # [F]
    w_2: np.ndarray     # [d, F]
    b_2: np.ndarray     # [d]
    mod: np.ndarray     # [6, d]: shift1, scale1, gate1, shift2, scale2, gate2
    # text cross-attention (present when the workload has instruction tokens)
    w_qc: Optional[np.ndarray] = None    # [d, d]
    b_qc: Optional[np.ndarray] = None    # [d]
    w_kvc: Optional[np.ndarray] = None   # [2d, d]  rows: K, V
    b_kvc: Optional[np.ndarray] = None   # [2d]
    w_oc: Optional[np.ndarray] = None    # [d, d]
    b_oc: Optional[np.ndarray] = None    # [d]


def make_weights(wl: Workload, seed: int = SEED_WEIGHTS) -> List[LayerWeights]:
    """Per-layer weights ~ N(0, 0.02); modulation shift/scale ~ N(0, 0.02) and
    gates 1 + N(0, 0.02) so both residual branches stay visible."""
    d, F = wl.d_model, wl.d_ffn
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(wl.n_layers):
        w_qkv = _normal(rng, (3 * d, d), 0.02)
        b_qkv = _normal(rng, (3 * d,), 0.02)
        w_o = _normal(rng, (d, d), 0.02)
        b_o = _normal(rng, (d,), 0.02)
        w_1 = _normal(rng, (F, d), 0.02)
        b_1 = _normal(rng, (F,), 0.02)
        w_2 = _normal(rng, (d, F), 0.02)
        b_2 = _normal(rng, (d,), 0.02)
        mod = _normal(rng, (6, d), 0.02)
        mod[2] += 1.0
        mod[5] += 1.0
        out.append(LayerWeights(*[_store(wl, a) for a in
                                  (w_qkv, b_qkv, w_o, b_o, w_1, b_1, w_2, b_2, mod)]))
    if wl.n_text > 0:
        # a generator of its own, so the self-attention / MLP weights above do
        # not depend on whether the workload has a text cross-attention
        rc = np.random.default_rng([seed, SEED_TEXT_WEIGHTS])
        for lw in out:
            lw.w_qc = _store(wl, _normal(rc, (d, d), 0.02))
            lw.b_qc = _store(wl, _normal(rc, (d,), 0.02))
            lw.w_kvc = _store(wl, _normal(rc, (2 * d, d), 0.02))
            lw.b_kvc = _store(wl, _normal(rc, (2 * d,), 0.02))
            lw.w_oc = _store(wl, _normal(rc, (d, d), 0.02))
            lw.b_oc = _store(wl, _normal(rc, (d,), 0.02))
    return out


def make_patch_embed(wl: Workload, seed: int = SEED_PATCH) -> np.ndarray:
    """W_pe [d, 16] ~ N(0, 0.02): the stand-in for the VAE + patch embedding."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (wl.d_model, LATENT_CH), 0.02)


def _paste(grid: np.ndarray, tex: np.ndarray, r0: int, c0: int) -> None:
    """Overwrite grid[r0:r0+h, c0:c0+w] with tex, clipped to the grid."""
    R, C = grid.shape[:2]
    h, w = tex.shape[:2]
    ra, rb = max(r0, 0), min(r0 + h, R)
    ca, cb = max(c0, 0), min(c0 + w, C)
    if ra >= rb or ca >= cb:
        return
    grid[ra:rb, ca:cb] = tex[ra - r0:rb - r0, ca - c0:cb - c0]


def _bounce(p0: int, v: int, t: int, lo: int, hi: int) -> int:
    """Position after t steps of velocity v, reflecting inside [lo, hi]."""
    span = hi - lo
    if span <= 0:
        return lo
    x = (p0 - lo) + v * t
    period = 2 * span
    x %= period
    return lo + (x if x <= span else period - x)


class LatentSource:
    """Produces the latent [views, rows, cols, 16] of episode e at chunk t."""

    def __init__(self, wl: Workload, episode: int = 0):
        self.wl = wl
        self.e = episode
        V, R, C = wl.views, wl.rows, wl.cols
        rng = np.random.default_rng(SEED_LATENT + episode)
        self.base = _normal(rng, (V, R, C, LATENT_CH))
        kind = wl.latent
        if kind == "blob":
            self.tex = _normal(rng, (4, 4, LATENT_CH))
        elif kind == "patch":
            r0, r1 = int(R * 22 / 64), int(R * 42 / 64)
            c0, c1 = int(C * 22 / 64), int(C * 42 / 64)
            self.region = (r0, r1, c0, c1)
            self.drift = _normal(rng, (r1 - r0, c1 - c0, LATENT_CH), 0.25)
        elif kind == "stack":
            self.ee = _normal(rng, (6, 6, LATENT_CH))
            self.obj = _normal(rng, (4, 4, LATENT_CH))
            self.offsets = [(0, 0), (3, -4), (-3, 5)]
        elif kind == "episodes":
            self.ee = _normal(rng, (min(8, R), min(8, C), LATENT_CH))
            self.obj = _normal(rng, (min(6, R), min(6, C), LATENT_CH))
            self.motion = []
            for _v in range(V):
                starts = rng.integers(0, [R, C, R, C])
                vel = rng.choice(np.array([-2, -1, 1, 2]), size=4)
                self.motion.append((starts, vel))
        else:
            raise ValueError(kind)

    def latent(self, t: int) -> np.ndarray:
        wl = self.wl
        lat = self.base.copy()
        R, C = wl.rows, wl.cols
        if wl.latent == "blob":
            _paste(lat[0], self.tex, 2 + t, 3 + t)
        elif wl.latent == "patch":
            r0, r1, c0, c1 = self.region
            lat[0, r0:r1, c0:c1] += np.float32(t) * self.drift
        elif wl.latent == "stack":
            er, ec = 4 + t, 6 + 2 * t
            for v in range(wl.views):
                dr, dc = self.offsets[v % len(self.offsets)]
                _paste(lat[v], self.ee, er + dr, ec + dc)
                if t < 8:
                    _paste(lat[v], self.obj, 14 + dr, 30 + dc)
                else:
                    _paste(lat[v], self.obj, er + 1 + dr, ec + 1 + dc)
        elif wl.latent == "episodes":
            for v in range(wl.views):
                (sr, sc, orr, oc), (vr, vc, ovr, ovc) = self.motion[v]
                eh, ew = self.ee.shape[:2]
                oh, ow = self.obj.shape[:2]
                _paste(lat[v], self.ee, _bounce(sr, vr, t, 0, R - eh), _bounce(sc, vc, t, 0, C - ew))
                _paste(lat[v], self.obj, _bounce(orr, ovr, t, 0, R - oh), _bounce(oc, ovc, t, 0, C - ow))
        return lat


def tokens_from_latent(wl: Workload, lat: np.ndarray, w_pe: np.ndarray) -> np.ndarray:
    """Flatten [views, rows, cols, 16] with token id (v*rows + r)*cols + c and
    apply the seeded patch embedding: z = latent @ W_pe^T, stored in the
    workload's dtype."""
    flat = lat.reshape(wl.n_tokens, LATENT_CH).astype(np.float64)
    z = flat @ w_pe.astype(np.float64).T
    return _store(wl, z.astype(np.float32))


def make_queries(wl: Workload, t: int, episode: int = 0) -> np.ndarray:
    """Action-query stand-ins Qa [L, A, d] ~ N(0, 1), drawn per (episode,
    chunk, layer)."""
    rng = np.random.default_rng([SEED_QUERY + episode, t])
    return _store(wl, np.stack([_normal(rng, (wl.n_action, wl.d_model))
                                for _ in range(wl.n_layers)]))


def make_initial_ages(wl: Workload, episode: int = 0) -> np.ndarray:
    """Ages after the dense chunk: zeros, or U{0..G} for workloads that start
    mid-rollout (so that some tokens are already forced)."""
    if not wl.random_initial_ages:
        return np.zeros(wl.n_tokens, dtype=np.int32)
    rng = np.random.default_rng([SEED_AGES, episode])
    return rng.integers(0, wl.age_bound + 1, size=wl.n_tokens).astype(np.int32)


@dataclass
class Rollout:
    """All inputs of a rollout: weights, and per episode the token
    embeddings z[t] and action queries Qa[t] for t = 0..chunks-1."""
    wl: Workload
    weights: List[LayerWeights]
    z: List[List[np.ndarray]]            # [episode][chunk] -> [N, d]
    qa: List[List[Optional[np.ndarray]]]  # [episode][chunk] -> [L, A, d] (None at t=0)
    ages0: List[np.ndarray]              # [episode] -> [N] int32
    text: Optional[List[np.ndarray]] = None   # [episode] -> [T, d] instruction embeddings


def make_text(wl: Workload, episode: int = 0) -> np.ndarray:
    """Instruction embeddings E [T, d] ~ N(0, 1) (a stand-in for the text
    encoder's output), fixed for the episode."""
    rng = np.random.default_rng([SEED_TEXT, episode])
    return _store(wl, _normal(rng, (wl.n_text, wl.d_model)))


def make_rollout(wl: Workload, chunks: Optional[int] = None) -> Rollout:
    T = wl.chunks if chunks is None else chunks
    weights = make_weights(wl)
    w_pe = make_patch_embed(wl)
    zs, qs, ages = [], [], []
    for e in range(wl.batch):
        src = LatentSource(wl, e)
        zs.append([tokens_from_latent(wl, src.latent(t), w_pe) for t in range(T)])
        qs.append([None] + [make_queries(wl, t, e) for t in range(1, T)])
        ages.append(make_initial_ages(wl, e))
    text = [make_text(wl, e) for e in range(wl.batch)] if wl.n_text > 0 else None
    return Rollout(wl, weights, zs, qs, ages, text)
