"""The paged forward's entry point that allocates nothing
(dsa_sparse_mla_fwd_paged_noalloc), through the C ABI, against the paged
entry point with a caller workspace on the same inputs.

Both run the same kernels with the same split count, so the outputs must be
bitwise equal; the first call is also checked against the oracle at the
forward's tolerance (O atol = rtol = 2e-2, LSE atol = rtol = 1e-3). Two calls
in a row, the second with a smaller input, exercise the shared scratch array
keeping the last call's contents.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import sparse_mla_fwd_paged_ref

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dsa():
    import dsa_sparse_mla_amd as dsa
    return dsa


def _inputs(num_seqs, seed):
    d = workloads.make_paged(num_seqs=num_seqs, q_per_seq=6, min_len=1500, max_len=6000, topk=2048,
                             seed=seed)
    return {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}, d


def _both(dev, splits):
    dsa = _dsa()
    T, H = dev["q"].shape[:2]
    args = (dev["q"], dev["kv_pages"], dev["page_table"], dev["seq_lens"], dev["indices"],
            dev["sm_scale"], dev["q_per_seq"])
    o_ref = torch.full((T, H, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    l_ref = torch.full((T, H), 7.0, dtype=torch.float32, device=DEV)
    dsa.sparse_mla_fwd_paged(*args, out=o_ref, lse=l_ref, num_splits=splits)
    o = torch.full((T, H, 512), -3.0, dtype=torch.bfloat16, device=DEV)
    l = torch.full((T, H), -3.0, dtype=torch.float32, device=DEV)
    dsa.sparse_mla_fwd_paged_noalloc(*args, out=o, lse=l, num_splits=splits)
    torch.cuda.synchronize()
    return o_ref, l_ref, o, l


def test_noalloc_matches_the_workspace_entry_point_twice():
    dsa = _dsa()
    # first call: 64 sequences x 6 tokens, the decode workload's batch (two splits)
    dev, host = _inputs(64, seed=21)
    T, H = dev["q"].shape[:2]
    splits, nbytes = dsa.workspace_size(T, H, 2048, 0)
    assert splits == 2 and 0 < nbytes <= 32 << 20
    o_ref, l_ref, o, l = _both(dev, 0)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    ro, rl = sparse_mla_fwd_paged_ref(host["q"].float().numpy(), host["kv_pages"].float().numpy(),
                                      host["page_table"].numpy(), host["seq_lens"].numpy(),
                                      host["indices"].numpy(), host["sm_scale"], host["q_per_seq"])
    on, ln = o.float().cpu().numpy(), l.cpu().numpy()
    assert np.all(np.abs(on - ro) <= 2e-2 + 2e-2 * np.abs(ro))
    assert np.all(np.abs(ln - rl) <= 1e-3 + 1e-3 * np.abs(rl))
    # second call, smaller: 5 sequences with 4 forced splits; the scratch still
    # holds the first call's partials, which this call must not read
    dev2, _ = _inputs(5, seed=22)
    o_ref, l_ref, o, l = _both(dev2, 4)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_unsplit_and_oversized():
    dsa = _dsa()
    dev, _ = _inputs(3, seed=23)
    o_ref, l_ref, o, l = _both(dev, 1)   # no split: the scratch is not used
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    # partials beyond the scratch size are refused before any launch:
    # 3 x 6 tokens x 32 splits x 8 heads x 2056 bytes = 9.5 MB fits, so ask
    # for more heads' worth via 128 heads x 32 splits = 151 MB
    d = workloads.make_paged(num_seqs=3, q_per_seq=6, num_heads=128, min_len=1500, max_len=6000,
                             topk=2048, seed=24)
    dv = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    T, H = dv["q"].shape[:2]
    out = torch.zeros((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((T, H), dtype=torch.float32, device=DEV)
    _, need = dsa.workspace_size(T, H, 2048, 32)
    assert need > 32 << 20
    with pytest.raises(dsa.DsaError) as e:
        dsa.sparse_mla_fwd_paged_noalloc(dv["q"], dv["kv_pages"], dv["page_table"], dv["seq_lens"],
                                         dv["indices"], dv["sm_scale"], dv["q_per_seq"], out=out,
                                         lse=lse, num_splits=32)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0   # nothing was launched
