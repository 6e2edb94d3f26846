"""One context-parallel rank's share of causal THD attention on MI355X (gfx950).

The computation lives in libcpthd.so (hand-written HIP kernels behind the C ABI
of include/cpthd.h); ``api`` is its Python binding.  Importing the package does
not load the library; the first call does, and raises if it was not built.
"""
from .api import (  # noqa: F401
    DUAL_CHUNK_SWAP, NO_LOAD_BALANCE, PACKED_SUPER_SEQUENCE, AttnPlan, CPAttention, HipEvents, attention, attn_bwd, attn_fwd,
    check_dev_status, cpthd_attn_bwd, cpthd_attn_bwd_allgathered, cpthd_attn_bwd_timed, cpthd_attn_bwd_noalloc, STATIC_SCRATCH_BYTES, cpthd_attn_fwd, cpthd_attn_fwd_allgathered,
    cpthd_attn_fwd_timed, Layout, cpthd_attn_plan, cpthd_attn_workspace_bytes,
    cpthd_attn_workspace_min_bytes,
    cpthd_gather_rows, cpthd_partition_indices, cpthd_reorder_kv, gather_rows, get_batch_on_this_cp_rank,
    partition_indices, reorder_kv,
)
