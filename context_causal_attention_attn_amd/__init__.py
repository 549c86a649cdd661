"""One context-parallel rank's causal attention share on MI355X (gfx950).

The computation runs in the HIP library libcpattn.so (built in-tree by
``context_causal_attention_attn_amd.build``); this package is its Python
binding. Importing the binding does not load the library; the first call
does, and raises ImportError if the library has not been built.
"""
from .api import (  # noqa: F401
    cp_attn_share_positions,
    cp_attn_validate,
    cp_attn_share_pairs,
    cp_attn_workspace_bytes,
    cp_attn_plan_stats_fwd,
    cp_attn_fwd,
    cp_attn_bwd,
    cp_attn_bwd_timed,
    make_desc,
)
from .shares import Share, cut_share  # noqa: F401
from .ulysses import (cp_attn_ulysses_relayout, head_to_seq_pack, head_to_seq_unpack,  # noqa: F401
                      seq_to_head_pack, seq_to_head_unpack, ulysses_bwd_in_place, ulysses_fwd_in_place)
