"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product (the HIP library and its Python binding) never
imports, calls or links it, and it shares no code with them.

Every function here is pinned by ``tests/test_oracle_pins.py`` (printed masks and head
mapping, closed forms, invariants, finite-difference gradients, an fp64 library
cross-check); none is "parity unpinned".
"""
from .attention_fp64 import (  # noqa: F401
    kv_head_of, causal_keep_mask, keep_mask, alibi_bias, head_probabilities, head_forward, rows_forward,
    head_backward, forward, backward, gather_kvcache, forward_kvcache,
)
