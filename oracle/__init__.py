"""Float64 CPU oracle for Spatial Sparse Attention (SSA).  Test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it, and it shares no code
with the HIP library.
"""
from .ssa_oracle import (  # noqa: F401
    Partition, partition, pool, block_offsets, pool_conv, compress, compressed_block, select_topk, selected_block,
    window_partition, morton_codes, sfc_windows, window_cells, window_attention, combine,
    forward, forward_items, backward, rms_norm, rope_3d, qkv_gates,
    sdpa_dense,
)
