"""CPU oracle for attention-scored KV-cache eviction (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The library under
``decode_kv_cache_gqa_amd`` never imports it, and it never imports the
library: the two share no code.
"""
from .kvev_oracle import *  # noqa: F401,F403
