"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

from sparse_kv_refresh_amd import wamc

DEV = "cuda"


def act(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device=DEV, dtype=dtype if dtype is not None else t.dtype).contiguous()


def to_np(t):
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def max_rel(g, o):
    g, o = np.asarray(g, dtype=np.float64), np.asarray(o, dtype=np.float64)
    den = np.abs(o).max()
    return float(np.abs(g - o).max() / den) if den > 0 else float(np.abs(g - o).max())


def rel_l2(g, o):
    g, o = np.asarray(g, dtype=np.float64), np.asarray(o, dtype=np.float64)
    den = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / den) if den > 0 else float(np.linalg.norm(g - o))


def close(wl, g, o):
    """The parity bar: fp32 runs max relative error 1e-4 (per tensor, relative
    to the tensor's largest magnitude); bf16 runs relative L2 error 1e-2."""
    if wl.dtype == "fp32":
        e = max_rel(g, o)
        return e <= 1e-4, e
    e = rel_l2(g, o)
    return e <= 1e-2, e


def engine(wl, rollout, rows_cap=None):
    """An engine for the workload; with instruction tokens, the text
    keys/values are computed right away (as at episode onset)."""
    dims = wamc.dims_for(wl)
    weights = wamc.Engine.upload_weights(rollout.weights, act(wl), DEV)
    eng = wamc.Engine(dims, weights, rows_cap or wl.n_tokens, DEV)
    if getattr(rollout, "text", None) is not None:
        eng.text_kv(to_dev(np.stack(rollout.text), act(wl)))
    return eng


def batch_z(wl, rollout, t):
    return to_dev(np.stack([rollout.z[e][t] for e in range(wl.batch)]), act(wl))


def batch_q(wl, rollout, t):
    # [L, B, A, d]
    return to_dev(np.stack([rollout.qa[e][t] for e in range(wl.batch)], axis=1), act(wl))
