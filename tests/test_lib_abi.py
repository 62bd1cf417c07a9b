"""The C-ABI library loads on a machine without a GPU, exports every function
include/wamc.h declares, and rejects bad arguments on the host -- before any
device call -- with the documented status codes.  (No compute call is made
here; those run in the GPU tests.)"""
import ctypes

import pytest

from sparse_kv_refresh_amd import inputs as W
from sparse_kv_refresh_amd import wamc

FAKE = 0x100000          # aligned dummy device address, never dereferenced
MISALIGNED = FAKE + 4


def _dims(**kw):
    d = wamc.dims_for(W.preset("t_bf16_small"))
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_exports_every_declared_symbol():
    L = wamc.lib()
    names = wamc.header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    for n in ("wamc_score", "wamc_select", "wamc_refresh_layer", "wamc_prefill_chunk", "wamc_dense_prefill"):
        assert n in names


def test_version_and_status_strings():
    L = wamc.lib()
    assert L.wamc_version() == 100
    assert L.wamc_status_string(0) == b"ok"
    assert L.wamc_status_string(3) == b"workspace too small"


def test_workspace_bytes_grows_with_rows():
    d = _dims()
    a, b = wamc.workspace_bytes(d, 10), wamc.workspace_bytes(d, 300)
    assert 0 < a < b and b % 256 == 0


@pytest.mark.parametrize("field,value,code", [
    ("n_heads", 3, 1),          # d != H * dh
    ("d_model", 260, 1),
    ("batch", 0, 1),
    ("age_bound", -1, 1),
    ("dtype", 7, 1),
    ("ln_eps", 0.0, 1),
    ("head_dim", 64, 1),        # 2 * 64 != 256
    ("d_ffn", (1 << 22) + 8, 1),   # beyond the GEMMs' 32-bit in-tile offsets
    ("n_tokens", (1 << 30) + 1, 1),
])
def test_bad_dims(field, value, code):
    d = _dims(**{field: value})
    out = ctypes.c_size_t()
    st = wamc.lib().wamc_workspace_bytes(ctypes.byref(d), 1, ctypes.byref(out))
    assert st == code, wamc.lib().wamc_last_error()
    assert wamc.lib().wamc_last_error() != b""


def test_largest_ffn_accepted():
    d = _dims(d_ffn=1 << 22)
    out = ctypes.c_size_t()
    assert wamc.lib().wamc_workspace_bytes(ctypes.byref(d), 1, ctypes.byref(out)) == 0, wamc.lib().wamc_last_error()


def test_unsupported_head_dim_bf16():
    d = _dims(n_heads=4, head_dim=64)
    out = ctypes.c_size_t()
    assert wamc.lib().wamc_workspace_bytes(ctypes.byref(d), 1, ctypes.byref(out)) == 2


def test_select_argument_errors():
    L = wamc.lib()
    d = _dims()
    N = d.n_tokens
    # k out of range
    assert L.wamc_select(ctypes.byref(d), FAKE, FAKE, N + 1, N, FAKE, FAKE, None, None) == 1
    # rows_cap < k
    assert L.wamc_select(ctypes.byref(d), FAKE, FAKE, 50, 40, FAKE, FAKE, None, None) == 1
    # null / misaligned pointers
    assert L.wamc_select(ctypes.byref(d), None, FAKE, 5, N, FAKE, FAKE, None, None) == 1
    assert L.wamc_select(ctypes.byref(d), MISALIGNED, FAKE, 5, N, FAKE, FAKE, None, None) == 4
    assert b"score" in L.wamc_last_error()


def test_workspace_too_small():
    L = wamc.lib()
    d = _dims()
    need = wamc.workspace_bytes(d, d.n_tokens)
    lw = wamc.LayerW(*([FAKE] * 9))
    arr = (wamc.LayerW * d.n_layers)(*([lw] * d.n_layers))
    st = L.wamc_dense_prefill(ctypes.byref(d), arr, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, None)
    assert st == 3


def test_refresh_layer_errors():
    L = wamc.lib()
    d = _dims()
    lw = wamc.LayerW(*([FAKE] * 9))
    ws = wamc.workspace_bytes(d, 100)
    # layer out of range
    assert L.wamc_refresh_layer(ctypes.byref(d), 5, ctypes.byref(lw), FAKE, FAKE, FAKE, 100, FAKE, FAKE,
                                FAKE, ws, None) == 1
    # rows_cap beyond N
    assert L.wamc_refresh_layer(ctypes.byref(d), 0, ctypes.byref(lw), FAKE, FAKE, FAKE, d.n_tokens + 1, FAKE,
                                FAKE, FAKE, ws, None) == 1
    # a missing weight
    bad = wamc.LayerW(*([FAKE] * 8 + [None]))
    assert L.wamc_refresh_layer(ctypes.byref(d), 0, ctypes.byref(bad), FAKE, FAKE, FAKE, 100, FAKE, FAKE,
                                FAKE, ws, None) == 1


def test_prefill_chunk_override_needs_counts():
    L = wamc.lib()
    d = _dims()
    lw = wamc.LayerW(*([FAKE] * 9))
    arr = (wamc.LayerW * d.n_layers)(*([lw] * d.n_layers))
    ws = wamc.workspace_bytes(d, d.n_tokens)
    st = L.wamc_prefill_chunk(ctypes.byref(d), arr, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 10, FAKE, None,
                              FAKE, FAKE, None, None, d.n_tokens, FAKE, ws, None)
    assert st == 1 and b"k_eff_override" in L.wamc_last_error()


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        wamc._ptr(torch.zeros(4))


def test_union_entry_points_validate():
    L = wamc.lib()
    d = _dims()
    N = d.n_tokens
    assert L.wamc_select_union(ctypes.byref(d), FAKE, FAKE, FAKE, N + 1, 0, FAKE, FAKE, None, None) == 1
    assert L.wamc_select_union(ctypes.byref(d), FAKE, FAKE, FAKE, 3, -1, FAKE, FAKE, None, None) == 1
    assert L.wamc_select_union(ctypes.byref(d), None, FAKE, FAKE, 3, 3, FAKE, FAKE, None, None) == 1
    assert L.wamc_select_union(ctypes.byref(d), FAKE, MISALIGNED, FAKE, 3, 3, FAKE, FAKE, None, None) == 4
    lw = wamc.LayerW(*([FAKE] * 9))
    arr = (wamc.LayerW * d.n_layers)(*([lw] * d.n_layers))
    ws = wamc.workspace_bytes(d, N)
    # the union can hold every token: rows_cap must be N
    st = L.wamc_prefill_chunk_union(ctypes.byref(d), arr, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 10, 5, FAKE,
                                    FAKE, None, N - 1, FAKE, ws, None)
    assert st == 1 and b"rows_cap" in L.wamc_last_error()
    st = L.wamc_prefill_chunk_union(ctypes.byref(d), arr, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 10, 5, FAKE,
                                    FAKE, None, N, FAKE, ws - 1, None)
    assert st == 3


def test_text_cross_attention_validates():
    """With instruction tokens every layer needs its cross-attention weights
    and text caches; wamc_text_kv needs n_text > 0."""
    L = wamc.lib()
    d = _dims(n_text=12)
    lw = wamc.LayerW(*([FAKE] * 9 + [None] * 8))
    ws = wamc.workspace_bytes(d, 100)
    assert L.wamc_refresh_layer(ctypes.byref(d), 0, ctypes.byref(lw), FAKE, FAKE, FAKE, 100, FAKE, FAKE,
                                FAKE, ws, None) == 1
    assert b"w_qc" in L.wamc_last_error()
    full = wamc.LayerW(*([FAKE] * 17))
    arr = (wamc.LayerW * d.n_layers)(*([full] * d.n_layers))
    d0 = _dims()
    assert L.wamc_text_kv(ctypes.byref(d0), arr, FAKE, FAKE, ws, None) == 1
    assert L.wamc_text_kv(ctypes.byref(d), arr, None, FAKE, ws, None) == 1
    d.n_text = -1
    assert L.wamc_workspace_bytes(ctypes.byref(d), 10, ctypes.byref(ctypes.c_size_t())) == 1


def test_noalloc_refuses_chunks_beyond_its_scratch():
    """The four-episode d=3072 chunk needs more workspace than the static
    scratch holds: refused on the host, before any device call."""
    L = wamc.lib()
    d = wamc.dims_for(W.preset("c5_large"))
    need = wamc.workspace_bytes(d, 4096)
    assert need > wamc.noalloc_scratch_bytes() == 256 << 20
    layers = (wamc.LayerW * d.n_layers)()
    P = ctypes.c_void_p(FAKE)
    st = L.wamc_prefill_chunk_noalloc(ctypes.byref(d), layers, P, P, P, None, P, P, P, 4096, None, None, P, P,
                                      None, None, 4096, None)
    assert st == 3
    assert b"static scratch" in L.wamc_last_error()
    # the 30-layer d=1536 chunk at the benchmark's row capacity fits
    assert wamc.workspace_bytes(wamc.dims_for(W.preset("c3_stack")), 2808) <= wamc.noalloc_scratch_bytes()


def test_prefill_chunk_refuses_a_capacity_the_forced_tokens_may_overflow():
    """With the library selecting, rows_cap must hold the N - k tokens the
    age bound can force (N when G = 0), so no forced token is left out."""
    L = wamc.lib()
    d = _dims()
    N = d.n_tokens
    lw = wamc.LayerW(*([FAKE] * 9))
    arr = (wamc.LayerW * d.n_layers)(*([lw] * d.n_layers))
    ws = wamc.workspace_bytes(d, N)

    def call(dims, k, rows_cap):
        return L.wamc_prefill_chunk(ctypes.byref(dims), arr, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, k, None,
                                    None, FAKE, FAKE, None, None, rows_cap, FAKE, ws, None)
    k = N // 4
    assert call(d, k, k) == 1 and b"force" in L.wamc_last_error()
    assert call(d, k, N - k - 1) == 1
    d0 = _dims(age_bound=0)
    assert call(d0, N - 10, N - 1) == 1
