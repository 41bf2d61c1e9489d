"""Rotated 4-bit paged KV cache for MI355X (gfx950).

The compute lives in the HIP library ``libkvq.so`` (sources in ``csrc/``); the
Python side only marshals arguments (``bit_kv_cache_02_amd.kvq``).  Importing
this package does not load the library; ``kvq`` loads it on first use and
raises if it is missing.
"""
