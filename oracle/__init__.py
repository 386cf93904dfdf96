"""fp64 CPU oracle for ring attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (``ring_attention_ringattn_amd`` and its HIP
library) never imports it and shares no code with it; the only shared module
is ``synthetic``, which draws seeded random inputs and holds no attention
arithmetic.

* ``attention``: the plain definition, softmax(Q K^T * scale + mask) V with
  LSE, and its backward, in fp64 (pinned by tests/test_oracle_pins.py).
* ``ring``: the ring method emulated in fp64 (shards, circulating blocks,
  exact LSE merge); pinned against ``attention`` to 1e-12.
* ``dynamic_cp``: exhaustive Dynamic-CP planner for small instances (the
  optimum the product's heuristic solver is checked against); pinned by a
  hand-checked case in tests/test_dynamic_cp.py.

Every function is pinned by a test against closed forms, invariants, a
50-digit Decimal brute force or finite differences; none is "parity
unpinned".
"""
from .attention import (NONE, CAUSAL, DOC_CAUSAL, allowed_pairs, attention_backward,
                        attention_forward, count_allowed_pairs, docs_from_cu_seqlens)
from .ring import merge, ring_forward, shard_rows

__all__ = ["NONE", "CAUSAL", "DOC_CAUSAL", "allowed_pairs", "attention_forward",
           "attention_backward", "count_allowed_pairs", "docs_from_cu_seqlens",
           "merge", "ring_forward", "shard_rows"]
