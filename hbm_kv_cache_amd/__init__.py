"""hbm_kv_cache_amd -- tiered KV cache hot path for MI355X (gfx950).

The work happens in ``libkvt.so`` (hand-written HIP kernels behind a C ABI, declared in
``include/kvt.h``).  ``hbm_kv_cache_amd.kvt`` is the thin ctypes binding with the same names;
``hbm_kv_cache_amd.synth`` holds the seeded synthetic input generators.
"""
