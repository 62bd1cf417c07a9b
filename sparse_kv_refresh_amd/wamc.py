"""Thin ctypes binding of libwamc (include/wamc.h).

Argument marshalling only: every step of the path runs in the HIP library.
torch supplies device memory and the stream; tensors are passed as raw
device pointers.  There is no CPU fallback: if libwamc.so is missing the
first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# WAMC_LIB names another build of the library (for A/B measurements of build
# options); the in-tree libwamc.so otherwise
LIB_PATH = os.environ.get("WAMC_LIB") or os.path.join(PKG, "libwamc.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "wamc.h")

WAMC_FP32, WAMC_BF16 = 0, 1
STATUS = {0: "WAMC_OK", 1: "WAMC_ERR_ARG", 2: "WAMC_ERR_UNSUPPORTED", 3: "WAMC_ERR_WORKSPACE",
          4: "WAMC_ERR_ALIGN", 5: "WAMC_ERR_DEVICE"}


class WamcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("n_tokens", ctypes.c_int32), ("n_action", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("age_bound", ctypes.c_int32), ("ln_eps", ctypes.c_float), ("w_attn", ctypes.c_float),
                ("w_surprise", ctypes.c_float), ("n_text", ctypes.c_int32)]


LAYER_FIELDS = ("w_qkv", "b_qkv", "w_o", "b_o", "w_1", "b_1", "w_2", "b_2", "mod",
                "w_qc", "b_qc", "w_kvc", "b_kvc", "w_oc", "b_oc", "text_k", "text_v")


class LayerW(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_DP = ctypes.POINTER(Dims)
_LP = ctypes.POINTER(LayerW)

_SIGNATURES = {
    "wamc_version": ([], ctypes.c_int),
    "wamc_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "wamc_last_error": ([], ctypes.c_char_p),
    "wamc_workspace_bytes": ([_DP, _I, ctypes.POINTER(_SZ)], ctypes.c_int),
    "wamc_score": ([_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "wamc_select": ([_DP, _P, _P, _I, _I, _P, _P, _P, _P], ctypes.c_int),
    "wamc_gather": ([_DP, _P, _P, _P, _P, _I, _P, _P], ctypes.c_int),
    "wamc_refresh_layer": ([_DP, _I, _LP, _P, _P, _P, _I, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "wamc_prefill_chunk": ([_DP, _LP, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P],
                           ctypes.c_int),
    "wamc_prefill_chunk_noalloc": ([_DP, _LP, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _I, _P],
                                   ctypes.c_int),
    "wamc_select_union": ([_DP, _P, _P, _P, _I, _I, _P, _P, _P, _P], ctypes.c_int),
    "wamc_prefill_chunk_union": ([_DP, _LP, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _I, _P, _SZ, _P],
                                 ctypes.c_int),
    "wamc_text_kv": ([_DP, _LP, _P, _P, _SZ, _P], ctypes.c_int),
    "wamc_dense_prefill": ([_DP, _LP, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "wamc_timing_enable": ([ctypes.c_int], ctypes.c_int),
    "wamc_timing_count": ([], ctypes.c_int),
    "wamc_timing_get": ([ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_I),
                         ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
}

_lib = None


def lib():
    """Load libwamc.so (built by `python -m sparse_kv_refresh_amd.build_lib`)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libwamc.so not found at {LIB_PATH}; build it with "
                               "`python -m sparse_kv_refresh_amd.build_lib` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def header_functions() -> List[str]:
    """Names of the functions declared in include/wamc.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(wamc_\w+)\s*\(", text, flags=re.M)))


def _check(status: int):
    if status != 0:
        msg = lib().wamc_last_error().decode()
        raise WamcError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("libwamc takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libwamc takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def act_dtype(dims: Dims) -> torch.dtype:
    return torch.bfloat16 if dims.dtype == WAMC_BF16 else torch.float32


def make_dims(batch, n_layers, d_model, n_heads, d_ffn, n_tokens, n_action, dtype, age_bound,
              ln_eps=1e-6, w_attn=0.4, w_surprise=0.1, n_text=0) -> Dims:
    dt = {"fp32": WAMC_FP32, "bf16": WAMC_BF16}.get(dtype, dtype)
    return Dims(batch, n_layers, d_model, n_heads, d_model // n_heads, d_ffn, n_tokens, n_action, dt,
                age_bound, ln_eps, w_attn, w_surprise, n_text)


def dims_for(wl) -> Dims:
    """Dims of a workload description (sparse_kv_refresh_amd.inputs.Workload)."""
    return make_dims(wl.batch, wl.n_layers, wl.d_model, wl.n_heads, wl.d_ffn, wl.n_tokens, wl.n_action,
                     wl.dtype, wl.age_bound, wl.ln_eps, wl.w_attn, wl.w_surprise, getattr(wl, "n_text", 0))


def layer_struct(w: dict) -> LayerW:
    """One layer's pointers; the text cross-attention fields stay NULL when
    the dict has none."""
    return LayerW(*[_ptr(w.get(n)) for n in LAYER_FIELDS])


def _layers(layers: Sequence[dict]):
    arr = (LayerW * len(layers))(*[layer_struct(w) for w in layers])
    return arr


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def version() -> int:
    return lib().wamc_version()


def workspace_bytes(dims: Dims, rows_cap: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().wamc_workspace_bytes(ctypes.byref(dims), rows_cap, ctypes.byref(out)))
    return out.value


def score(dims, z, zref, q_act, k_cache, score_out, ws, mass_in=None, mass_out=None, surprise_out=None,
          stream=None):
    _check(lib().wamc_score(ctypes.byref(dims), _ptr(z), _ptr(zref), _ptr(q_act), _ptr(k_cache), _ptr(mass_in),
                            _ptr(score_out), _ptr(mass_out), _ptr(surprise_out), _ptr(ws), ws.numel(),
                            _stream(stream)))


def select(dims, score_t, age, k, rows_cap, idx, k_eff, n_forced=None, stream=None):
    _check(lib().wamc_select(ctypes.byref(dims), _ptr(score_t), _ptr(age), k, rows_cap, _ptr(idx), _ptr(k_eff),
                             _ptr(n_forced), _stream(stream)))


def gather(dims, z, zref, idx, k_eff, rows_cap, x, stream=None):
    _check(lib().wamc_gather(ctypes.byref(dims), _ptr(z), _ptr(zref), _ptr(idx), _ptr(k_eff), rows_cap, _ptr(x),
                             _stream(stream)))


def refresh_layer(dims, layer, w: dict, x, idx, k_eff, rows_cap, k_cache_l, v_cache_l, ws, stream=None):
    lw = layer_struct(w)
    _check(lib().wamc_refresh_layer(ctypes.byref(dims), layer, ctypes.byref(lw), _ptr(x), _ptr(idx), _ptr(k_eff),
                                    rows_cap, _ptr(k_cache_l), _ptr(v_cache_l), _ptr(ws), ws.numel(),
                                    _stream(stream)))


def prefill_chunk(dims, layers: Sequence[dict], z, zref, q_act, k_cache, v_cache, age, k, idx_out, k_eff_out,
                  rows_cap, ws, mass_in=None, idx_override=None, k_eff_override=None, score_out=None,
                  layer_out=None, stream=None, _layer_array=None):
    arr = _layer_array if _layer_array is not None else _layers(layers)
    _check(lib().wamc_prefill_chunk(ctypes.byref(dims), arr, _ptr(z), _ptr(zref), _ptr(q_act), _ptr(mass_in),
                                    _ptr(k_cache), _ptr(v_cache), _ptr(age), k, _ptr(idx_override),
                                    _ptr(k_eff_override), _ptr(idx_out), _ptr(k_eff_out), _ptr(score_out),
                                    _ptr(layer_out), rows_cap, _ptr(ws), ws.numel(), _stream(stream)))


def prefill_chunk_noalloc(dims, layers: Sequence[dict], z, zref, q_act, k_cache, v_cache, age, k, idx_out,
                          k_eff_out, rows_cap, mass_in=None, idx_override=None, k_eff_override=None,
                          score_out=None, layer_out=None, stream=None, _layer_array=None):
    """prefill_chunk with the library's static scratch in place of a
    workspace (for callers that cannot allocate device memory)."""
    arr = _layer_array if _layer_array is not None else _layers(layers)
    _check(lib().wamc_prefill_chunk_noalloc(ctypes.byref(dims), arr, _ptr(z), _ptr(zref), _ptr(q_act),
                                            _ptr(mass_in), _ptr(k_cache), _ptr(v_cache), _ptr(age), k,
                                            _ptr(idx_override), _ptr(k_eff_override), _ptr(idx_out),
                                            _ptr(k_eff_out), _ptr(score_out), _ptr(layer_out), rows_cap,
                                            _stream(stream)))


def noalloc_scratch_bytes() -> int:
    """Size of the static scratch behind prefill_chunk_noalloc (from the header)."""
    with open(HEADER) as f:
        m = re.search(r"#define\s+WAMC_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", f.read())
    return int(m.group(1)) << int(m.group(2))


def select_union(dims, mass, surprise, age, n_attn, n_surprise, idx, k_eff, n_forced=None, stream=None):
    _check(lib().wamc_select_union(ctypes.byref(dims), _ptr(mass), _ptr(surprise), _ptr(age), n_attn, n_surprise,
                                   _ptr(idx), _ptr(k_eff), _ptr(n_forced), _stream(stream)))


def prefill_chunk_union(dims, layers: Sequence[dict], z, zref, q_act, k_cache, v_cache, age, n_attn, n_surprise,
                        idx_out, k_eff_out, rows_cap, ws, mass_in=None, layer_out=None, stream=None,
                        _layer_array=None):
    arr = _layer_array if _layer_array is not None else _layers(layers)
    _check(lib().wamc_prefill_chunk_union(ctypes.byref(dims), arr, _ptr(z), _ptr(zref), _ptr(q_act), _ptr(mass_in),
                                          _ptr(k_cache), _ptr(v_cache), _ptr(age), n_attn, n_surprise, _ptr(idx_out),
                                          _ptr(k_eff_out), _ptr(layer_out), rows_cap, _ptr(ws), ws.numel(),
                                          _stream(stream)))


def text_kv(dims, layers: Sequence[dict], text, ws, stream=None, _layer_array=None):
    arr = _layer_array if _layer_array is not None else _layers(layers)
    _check(lib().wamc_text_kv(ctypes.byref(dims), arr, _ptr(text), _ptr(ws), ws.numel(), _stream(stream)))


def dense_prefill(dims, layers: Sequence[dict], z, zref, k_cache, v_cache, age, ws, layer_out=None, stream=None,
                  _layer_array=None):
    arr = _layer_array if _layer_array is not None else _layers(layers)
    _check(lib().wamc_dense_prefill(ctypes.byref(dims), arr, _ptr(z), _ptr(zref), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(age), _ptr(layer_out), _ptr(ws), ws.numel(), _stream(stream)))


def timing_enable(on: bool = True):
    _check(lib().wamc_timing_enable(1 if on else 0))


def timing_read() -> dict:
    """{kernel kind: (launches, total_ms)} recorded since timing was enabled."""
    L = lib()
    out = {}
    for i in range(L.wamc_timing_count()):
        name = ctypes.c_char_p()
        n = ctypes.c_int32()
        ms = ctypes.c_double()
        _check(L.wamc_timing_get(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)))
        out[name.value.decode()] = (n.value, ms.value)
    return out


# ---------------------------------------------------------------------------
# convenience: device state of a batch of episodes
# ---------------------------------------------------------------------------

class Engine:
    """Owns the per-episode device state (K/V cache, ages, reference
    embeddings), a workspace and the uploaded weights, and drives the five
    entry points.  All tensors live on `device`."""

    def __init__(self, dims: Dims, weights: Sequence[dict], rows_cap: int, device="cuda"):
        self.dims = dims
        self.device = torch.device(device)
        self.rows_cap = rows_cap
        B, L, N, d = dims.batch, dims.n_layers, dims.n_tokens, dims.d_model
        adt = act_dtype(dims)
        self.weights = [dict(w) for w in weights]
        T = dims.n_text
        if T > 0:
            # per-layer keys/values of the instruction, written by text_kv()
            self.text_k = torch.zeros((L, B, T, d), dtype=adt, device=self.device)
            self.text_v = torch.zeros((L, B, T, d), dtype=adt, device=self.device)
            for l, w in enumerate(self.weights):
                w["text_k"], w["text_v"] = self.text_k[l], self.text_v[l]
        self.layer_array = _layers(self.weights)
        self.k_cache = torch.zeros((L, B, N, d), dtype=adt, device=self.device)
        self.v_cache = torch.zeros((L, B, N, d), dtype=adt, device=self.device)
        self.zref = torch.zeros((B, N, d), dtype=adt, device=self.device)
        self.age = torch.zeros((B, N), dtype=torch.int32, device=self.device)
        self.idx = torch.full((B, N), -1, dtype=torch.int32, device=self.device)
        self.k_eff = torch.zeros((B,), dtype=torch.int32, device=self.device)
        self.score = torch.zeros((B, N), dtype=torch.float32, device=self.device)
        nbytes = max(workspace_bytes(dims, rows_cap), workspace_bytes(dims, N))
        self.ws = torch.empty((nbytes,), dtype=torch.uint8, device=self.device)

    @staticmethod
    def upload_weights(np_layers, dtype: torch.dtype, device="cuda") -> List[dict]:
        names = LAYER_FIELDS[:15]
        return [{n: torch.from_numpy(getattr(w, n)).to(device=device, dtype=dtype).contiguous() for n in names
                 if getattr(w, n, None) is not None} for w in np_layers]

    def text_kv(self, text, stream=None):
        """The instruction's keys/values for every layer (once per episode,
        before the dense chunk).  text: [B, T, d]."""
        text_kv(self.dims, self.weights, text, self.ws, stream=stream, _layer_array=self.layer_array)

    def dense(self, z, layer_out=None, stream=None):
        dense_prefill(self.dims, self.weights, z, self.zref, self.k_cache, self.v_cache, self.age, self.ws,
                      layer_out=layer_out, stream=stream, _layer_array=self.layer_array)

    def chunk(self, z, q_act, k, mass_in=None, idx_override=None, k_eff_override=None, layer_out=None,
              stream=None):
        prefill_chunk(self.dims, self.weights, z, self.zref, q_act, self.k_cache, self.v_cache, self.age, k,
                      self.idx, self.k_eff, self.rows_cap, self.ws, mass_in=mass_in, idx_override=idx_override,
                      k_eff_override=k_eff_override, score_out=self.score, layer_out=layer_out, stream=stream,
                      _layer_array=self.layer_array)

    def chunk_union(self, z, q_act, n_attn, n_surprise, mass_in=None, layer_out=None, stream=None):
        """A refresh chunk with the union rule (needs rows_cap == N)."""
        prefill_chunk_union(self.dims, self.weights, z, self.zref, q_act, self.k_cache, self.v_cache, self.age,
                            n_attn, n_surprise, self.idx, self.k_eff, self.rows_cap, self.ws, mass_in=mass_in,
                            layer_out=layer_out, stream=stream, _layer_array=self.layer_array)

    def snapshot(self):
        return {n: getattr(self, n).clone() for n in ("k_cache", "v_cache", "zref", "age")}

    def restore(self, snap):
        for n, t in snap.items():
            getattr(self, n).copy_(t)
