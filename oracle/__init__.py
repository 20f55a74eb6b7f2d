"""CPU oracle for TurboQuant-style KV compression and compressed-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product (the HIP library under ``compressed_kv_attention_tq_amd/`` and its
Python binding) never imports, links or calls it, and this package imports
nothing from the product.  The two share no code; the only thing both sides
consume is the seeded input generators in
``compressed_kv_attention_tq_amd/workloads.py``, which hold none of the
method's arithmetic.

See ``oracle/tq_oracle.py`` for the functions and the passages they follow.
"""

from .tq_oracle import *  # noqa: F401,F403
