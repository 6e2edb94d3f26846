"""CPU oracle (test infrastructure only: imported by tests, the smoke check and
the benchmark's CPU-baseline leg, never by the product path)."""
from .cpthd_oracle import (  # noqa: F401
    DUAL_CHUNK_SWAP, NO_LOAD_BALANCE, PACKED_SUPER_SEQUENCE, STRATEGIES, check_layout, token_map, partition_indices,
    all_gather, restore, batch_on_rank, useful_pairs, attn_fwd, attn_bwd,
)
