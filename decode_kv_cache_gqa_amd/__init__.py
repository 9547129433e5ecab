"""Attention-scored KV-cache eviction on MI355X (gfx950).

The compute path is the C-ABI shared library ``libkvev.so`` built from
``csrc/``; :mod:`decode_kv_cache_gqa_amd.kvev` is its thin ctypes binding.
:mod:`decode_kv_cache_gqa_amd.synth` holds the seeded synthetic workloads.
Importing the package loads nothing; the library is loaded on first use and
a missing or unloadable library raises.
"""
__all__ = ["kvev", "synth"]
