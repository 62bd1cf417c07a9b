"""sparse_kv_refresh_amd: staleness-bounded sparse KV-refresh prefill on
MI355X (gfx950).

Submodules:
  wamc       -- ctypes binding of libwamc.so (the HIP library, include/wamc.h)
  inputs     -- seeded synthetic workloads (weights, latents, queries)
  build_lib  -- builds libwamc.so in-tree with hipcc for gfx950
"""
__version__ = "1.0.0"
