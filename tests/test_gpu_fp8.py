"""GPU parity of the paged forward over an FP8 MLA cache
(dsa_sparse_mla_fwd_paged_fp8) against the FP8 oracle (oracle/fp8_cache_ref.py,
exact dequantisation in float64).

Tolerance: the forward's (O atol = rtol = 2e-2, LSE atol = rtol = 1e-3, and
the Frobenius relative error of O below 1e-2). The kernel rounds each scaled
latent value to bf16 (relative error <= 2^-9) before its MFMAs; with scores of
order 1 that moves a score by about 1e-3 at most, inside the LSE bound.

Exact cases: a cache whose latent codes carry scale 1 holds values that bf16
represents exactly, so the FP8 path must equal the bf16 paged path on the
same values bit for bit; page permutations leave the result bitwise
unchanged; an empty row gives O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import sparse_mla_fwd_paged_fp8_ref

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dsa():
    import dsa_sparse_mla_amd as dsa
    return dsa


def to_dev(d):
    return {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}


def run(d, **kw):
    dev = to_dev(d)
    out, lse = _dsa().sparse_mla_fwd_paged_fp8(dev["q"], dev["kv_pages"], dev["page_table"], dev["seq_lens"],
                                               dev["indices"], dev["sm_scale"], dev["q_per_seq"], **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def ref(d, rows=None):
    q = d["q"].float().numpy()
    idx = d["indices"].numpy()
    return sparse_mla_fwd_paged_fp8_ref(q, d["kv_pages"].cpu().numpy(), d["page_table"].numpy(),
                                        d["seq_lens"].numpy(), idx, d["sm_scale"], d["q_per_seq"])


def check(o, l, ro, rl, what):
    fin = np.isfinite(rl)
    assert np.all(np.abs(o - ro) <= 2e-2 + 2e-2 * np.abs(ro)), (what, np.abs(o - ro).max())
    assert np.array_equal(np.isfinite(l), fin), what
    assert np.all(np.abs(l[fin] - rl[fin]) <= 1e-3 + 1e-3 * np.abs(rl[fin])), (what, np.abs(l[fin] - rl[fin]).max())
    rel = np.linalg.norm(o - ro) / max(np.linalg.norm(ro), 1e-30)
    assert rel < 1e-2, (what, rel)


@pytest.mark.parametrize("H", [1, 8, 16, 17, 32])
def test_fp8_decode_heads(H):
    d = workloads.make_paged_fp8(num_seqs=5, q_per_seq=6, num_heads=H, min_len=700, max_len=4000, topk=2048,
                                 seed=40 + H)
    o, l = run(d)
    ro, rl = ref(d)
    check(o, l, ro, rl, f"fp8 H={H}")


@pytest.mark.parametrize("splits", [1, 2, 3, 8])
def test_fp8_splits_and_junk(splits):
    d = workloads.make_paged_fp8(num_seqs=4, q_per_seq=3, min_len=300, max_len=3000, topk=1500, seed=50 + splits)
    idx = d["indices"].clone()
    idx[0, :700] = -1                 # padding
    idx[1, 5] = 10 ** 8               # beyond the sequence
    idx[2, :] = -3                    # a row with no key
    idx[5, 7] = idx[5, 8]             # a duplicate entry
    d["indices"] = idx
    o, l = run(d, num_splits=splits)
    ro, rl = ref(d)
    assert np.all(o[2] == 0) and np.all(np.isneginf(l[2]))
    check(o, l, ro, rl, f"fp8 splits={splits}")


def test_fp8_equals_bf16_path_on_exact_values():
    """Codes with scale 1: every latent value is an e4m3 value, exact in bf16,
    and the FP8 path must reproduce the bf16 paged path bit for bit."""
    d = workloads.make_paged_fp8(num_seqs=4, q_per_seq=6, min_len=1000, max_len=3000, topk=2048, seed=61)
    raw = d["kv_pages"].clone()
    P, ps = raw.shape[:2]
    g = torch.Generator().manual_seed(3)
    codes = torch.randint(0, 256, (P, ps, 512), generator=g, dtype=torch.int32).to(torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                      # no NaN code
    raw[..., :512] = codes
    raw[..., 512:528] = torch.ones((P, ps, 4), dtype=torch.float32).view(torch.uint8)
    d["kv_pages"] = raw
    lat = codes.view(torch.float8_e4m3fn).to(torch.bfloat16)
    rope = raw[..., 528:].contiguous().view(torch.bfloat16)
    kv_bf16 = torch.cat([lat, rope], dim=-1)
    o8, l8 = run(d)
    dev = to_dev(d)
    out, lse = _dsa().sparse_mla_fwd_paged(dev["q"], kv_bf16.to(DEV), dev["page_table"], dev["seq_lens"],
                                           dev["indices"], d["sm_scale"], d["q_per_seq"])
    torch.cuda.synchronize()
    assert np.array_equal(o8, out.float().cpu().numpy())
    assert np.array_equal(l8, lse.cpu().numpy())


def test_fp8_page_permutation_bitwise_and_strided_rows():
    """Physical pages permuted (and the table with them): bitwise equal. Rows
    stored 688 bytes apart and pages padded: same result."""
    d = workloads.make_paged_fp8(num_seqs=3, q_per_seq=6, min_len=2000, max_len=5000, topk=2048, seed=71)
    o1, l1 = run(d)
    P = d["kv_pages"].shape[0]
    perm = torch.from_numpy(np.random.default_rng(1).permutation(P))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P)
    d2 = dict(d)
    d2["kv_pages"] = d["kv_pages"][inv]
    table = d["page_table"].clone()
    ok = table >= 0
    table[ok] = perm[table[ok].long()].int()
    d2["page_table"] = table
    o2, l2 = run(d2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    wide = torch.zeros((P + 0, d["kv_pages"].shape[1] + 1, 688), dtype=torch.uint8)
    wide[:, :-1, :656] = d["kv_pages"]
    d3 = dict(d)
    d3["kv_pages"] = wide[:, :-1, :]                             # row stride 688, page stride 65 rows
    o3, l3 = run(d3)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_fp8_rejects_more_than_32_heads():
    d = workloads.make_paged_fp8(num_seqs=1, q_per_seq=2, num_heads=64, min_len=100, max_len=200, topk=64)
    with pytest.raises(_dsa().DsaError) as e:
        run(d)
    assert e.value.status == 2


def test_fp8_full_decode_sampled():
    """The decode workload's shape (64 sequences x 6 tokens, contexts up to
    65536, 8 heads) with the FP8 cache, in the launch configuration bench.py
    times; 48 sampled tokens (whole sequences) against the oracle."""
    d = workloads.make_paged_fp8(device="cuda")
    out, lse = _dsa().sparse_mla_fwd_paged_fp8(d["q"], d["kv_pages"], d["page_table"], d["seq_lens"],
                                               d["indices"], d["sm_scale"], d["q_per_seq"])
    torch.cuda.synchronize()
    Q = d["q_per_seq"]
    seqs = [0, 17, 40, 63]
    rows = np.concatenate([np.arange(s * Q, (s + 1) * Q) for s in seqs])
    # only the sampled sequences' pages, renumbered, go to the oracle
    table = d["page_table"][seqs].cpu().numpy()
    used = np.unique(table[table >= 0])
    remap = np.full(d["kv_pages"].shape[0], -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    small_table = np.where(table >= 0, remap[np.maximum(table, 0)], -1).astype(np.int32)
    pages = d["kv_pages"][torch.from_numpy(used).to(d["kv_pages"].device)].cpu().numpy()
    ro, rl = sparse_mla_fwd_paged_fp8_ref(d["q"][rows].float().cpu().numpy(), pages, small_table,
                                          d["seq_lens"][seqs].cpu().numpy(),
                                          d["indices"][rows].cpu().numpy(), d["sm_scale"], Q)
    check(out[rows].float().cpu().numpy(), lse[rows].cpu().numpy(), ro, rl, "fp8 decode full")
