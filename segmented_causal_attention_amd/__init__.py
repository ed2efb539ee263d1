"""Segmented causal attention for AMD Instinct MI355X (gfx950).

The compute path lives in ``libsegattn.so`` (hand-written HIP kernels behind
the C ABI declared in ``include/segattn.h``); ``binding`` marshals torch
tensors and numpy item tables into those calls.  Build the library with
``python -m segmented_causal_attention_amd.build``.
"""

from .binding import (  # noqa: F401
    SegattnError,
    make_shape,
    segattn_bwd,
    segattn_bwd_noalloc,
    segattn_bwd_preprocess,
    segattn_bwd_workspace,
    segattn_chunk_varlen,
    segattn_copy_rows,
    segattn_fwd,
    segattn_fwd_prepare,
    segattn_fwd_workspace,
    segattn_merge,
    segattn_offload_plan,
    segattn_partition,
    segattn_partition_varlen,
    segattn_ring_items,
    segattn_stream_order,
    segattn_version,
)
