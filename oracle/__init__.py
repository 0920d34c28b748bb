"""CPU oracle for the DSA sparse MLA forward and backward, and the top-k index selection.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this package:
only the test suite, the smoke check and the CPU-baseline leg of the benchmark
call it. It shares no code with the HIP library.
"""
from .sparse_mla_ref import (  # noqa: F401
    DQK,
    DV,
    map_paged_indices,
    sparse_mla_fwd_ref,
    sparse_mla_fwd_paged_ref,
)
from .bwd_ref import sparse_mla_bwd_ref  # noqa: F401,E402
from .topk_ref import topk_indices_ref  # noqa: F401,E402
from .fp8_cache_ref import dequantize_rows, e4m3_to_float, sparse_mla_fwd_paged_fp8_ref  # noqa: F401,E402
