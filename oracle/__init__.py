"""TEST INFRASTRUCTURE ONLY: the plain fp64 CPU oracle for one context-parallel
rank's causal attention share.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package. The product path
(the HIP library and its Python binding) never does, and shares no code with it.

Parity status of each function is stated in ``oracle/cp_share.py``'s header.
"""
from .cp_share import (  # noqa: F401
    kv_head_of,
    visible,
    share_chunks,
    chunk_row_positions,
    attention_rows,
    attention_rows_bwd,
    contiguous_share,
    head_tail_share,
    ulysses_share,
    hybrid_share,
    share_pairs,
)
