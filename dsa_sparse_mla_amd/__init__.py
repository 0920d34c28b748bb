"""DSA sparse MLA forward (and backward) on AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind a C ABI
(include/dsa_sparse_mla.h, built into libdsa_sparse_mla.so next to this file).
This package only marshals torch tensors into that ABI:

    out, lse = sparse_mla_fwd(q, kv, indices, sm_scale)
    out, lse = sparse_mla_fwd_paged(q, kv_pages, page_table, seq_lens, indices,
                                    sm_scale, q_per_seq)
    dq, dkv = sparse_mla_bwd(q, kv, indices, sm_scale, out, lse, dout)
    indices = topk_indices(scores, key_start, key_end, topk)
"""
from .binding import (  # noqa: F401
    DQK,
    DV,
    LIB_PATH,
    bwd_workspace_size,
    DsaError,
    lib,
    sparse_mla_bwd,
    sparse_mla_fwd,
    sparse_mla_fwd_paged,
    sparse_mla_fwd_paged_fp8,
    sparse_mla_fwd_paged_noalloc,
    topk_indices,
    workspace_size,
)

__all__ = ["sparse_mla_fwd", "topk_indices", "sparse_mla_fwd_paged", "sparse_mla_bwd", "workspace_size", "bwd_workspace_size", "DsaError", "lib"]
