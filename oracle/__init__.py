"""Oracle for segmented causal attention: plain, slow, float64 / exact-integer
reference implementations written from the source pages.

This package is TEST INFRASTRUCTURE. Only the test-suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (the HIP library and its Python binding) never imports,
links or calls anything here, and nothing here imports the product path.

Modules
-------
planner    -- FLOPs-balanced segment boundaries, varlen slicing and ring-order
              work items (exact integer arithmetic).
attention  -- causal softmax attention forward / backward in float64, the
              log-sum-exp merge of partial results, and the segmented
              (item-by-item) evaluation used to check the identity
              "segmented + merged == unsegmented".
offload    -- the sequence-aware offload plan (ratios alpha_i and the GPU
              memory recurrence) in float64.
chunking   -- workload-balanced chunking of a variable-length batch (mesh
              from the longest sequence, mesh cuts, best-fit-decreasing
              packing of tails and short sequences) in float64.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, library routines, finite differences and exact
invariants); none is "parity unpinned".
"""

from .planner import (  # noqa: F401
    tri,
    boundary,
    segment_work,
    partition,
    partition_varlen,
    ring_items,
    ring_steps,
)
from .attention import (  # noqa: F401
    kv_head_of,
    attention_fwd,
    attention_partial,
    merge,
    segmented_fwd,
    attention_bwd,
    segmented_bwd,
    attention_rows,
    attention_rows_bwd,
    attention_keys_bwd,
)
from .offload import plan_offload, offload_rows  # noqa: F401,E402
from .chunking import chunk, chunk_items  # noqa: F401,E402
