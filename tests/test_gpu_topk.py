"""GPU parity of the top-k index selection (dsa_topk_indices) against the
oracle (oracle/topk_ref.py). Integer work: every row must be bit-exact.

Cases: normal, tie-heavy and special-valued scores (inf, NaN, +-0); rows
shorter than, equal to and just above topk; empty and clipped ranges; rows
longer than the kernel's LDS key cache; strided scores and index rows; no
scores at all; the full-size wide and packed-varlen prefill ranges and the
decode contexts; and the chain scores -> top-k -> sparse forward against the
two oracles.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import topk_indices_ref, sparse_mla_fwd_ref

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dsa():
    import dsa_sparse_mla_amd as dsa
    return dsa


def run(scores, ks, ke, topk, num_cols=None):
    dsa = _dsa()
    sd = scores.to(DEV) if scores is not None else None
    got = dsa.topk_indices(sd, ks.to(DEV), ke.to(DEV), topk, num_cols=num_cols)
    torch.cuda.synchronize()
    return got.cpu().numpy()


def ref(scores, ks, ke, topk, num_cols=None):
    s = scores.cpu().numpy() if scores is not None else None
    return topk_indices_ref(s, ks.numpy(), ke.numpy(), topk, num_cols=num_cols)


def _i32(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.int32)


@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
@pytest.mark.parametrize("topk", [1, 7, 64, 2048])
def test_topk_random_ranges(kind, topk):
    T, C = 96, 5000
    scores = workloads.index_scores(T, C, seed=10 + topk, kind=kind)
    rng = np.random.default_rng(topk)
    ks = rng.integers(-50, C, T)
    ke = ks + rng.integers(-20, 4 * topk + 40, T)
    ke[:4] = ks[:4] + np.array([topk, topk + 1, topk - 1, 0])     # at, above, below topk; empty
    ks, ke = _i32(ks), _i32(ke)
    got = run(scores, ks, ke, topk)
    want = ref(scores, ks, ke, topk)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n", [16384, 16385, 70000])
def test_topk_long_rows(n):
    """At and past the LDS key cache (16384 candidates): the longer rows read
    their scores again in every pass."""
    T, topk = 6, 2048
    scores = workloads.index_scores(T, n + 7, seed=n, kind="normal")
    scores[1] = torch.floor(scores[1] * 3)                      # ties inside a long row
    ks = _i32([0, 0, 7, 3, 0, 100])
    ke = _i32([n, n, n + 7, n - 5, n + 7, n - 1])
    got = run(scores, ks, ke, topk)
    assert np.array_equal(got, ref(scores, ks, ke, topk))


def test_topk_strided_and_wide_topk():
    """Score rows wider than num_cols, index rows wider than topk; topk 4500."""
    T, C, topk = 40, 9000, 4500
    base = workloads.index_scores(T, C + 64, seed=3, kind="ties")
    scores = base[:, :C]                                          # row stride C + 64
    rng = np.random.default_rng(5)
    ks = _i32(rng.integers(0, 1000, T))
    ke = _i32(np.asarray(ks) + rng.integers(0, 8000, T))
    dsa = _dsa()
    big = torch.full((T, topk + 9), 12345, dtype=torch.int32, device=DEV)
    view = big[:, :topk]
    dsa.topk_indices(scores.to(DEV), ks.to(DEV), ke.to(DEV), topk, indices=view)
    torch.cuda.synchronize()
    out = big.cpu().numpy()
    assert np.array_equal(out[:, :topk], ref(scores.contiguous(), ks, ke, topk))
    assert np.all(out[:, topk:] == 12345)


def test_topk_without_scores():
    """No scores: short rows are written whole (the scoring skip), longer rows
    select nothing."""
    T, C, topk = 8, 300, 64
    ks = _i32([0, 10, 0, 5, 299, 0, 50, 0])
    ke = _i32([64, 40, 65, 4, 300, 0, 120, 300])
    got = run(None, ks, ke, topk, num_cols=C)
    assert np.array_equal(got, ref(None, ks, ke, topk, num_cols=C))
    assert np.all(got[2] == -1) and np.array_equal(got[0], np.arange(64))


def test_topk_short_prefill_is_all_causal_keys():
    """The short prefill (64 tokens, topk 2048): every token selects its whole
    causal prefix, unscored."""
    ks, ke = workloads.causal_ranges(None, 64)
    got = run(None, ks, ke, 2048, num_cols=64)
    for t in range(64):
        assert np.array_equal(got[t, :t + 1], np.arange(t + 1)) and np.all(got[t, t + 1:] == -1)


def test_topk_full_wide_prefill():
    """8192 causal rows of up to 8192 candidates, topk 2048 (the wide
    workload's ranges): every row bit-exact."""
    T = 8192
    scores = workloads.index_scores(T, T, seed=31, kind="normal", device="cuda")
    ks, ke = workloads.causal_ranges(None, T)
    got = run(scores, ks, ke, 2048)
    want = ref(scores.cpu(), ks, ke, 2048)
    assert np.array_equal(got, want)


def test_topk_full_varlen16k_sampled():
    """Packed 16384-token documents (the varlen workload's cu_seqlens):
    candidates limited to the token's own document; 1024 sampled rows."""
    T = 16384
    cu = workloads.varlen_cu_seqlens("varlen16k")
    assert np.array_equal(cu, workloads.make_flat("varlen16k", num_tokens=T, num_heads=1, topk=1)["cu_seqlens"])
    ks, ke = workloads.causal_ranges(cu, T)
    scores = workloads.index_scores(T, T, seed=41, kind="ties", device="cuda")
    got = run(scores, ks, ke, 2048)
    rows = np.random.default_rng(0).choice(T, 1024, replace=False)
    sc = scores[torch.from_numpy(rows).to(scores.device)].cpu()
    want = topk_indices_ref(sc.numpy(), ks.numpy()[rows], ke.numpy()[rows], 2048, num_cols=T)
    assert np.array_equal(got[rows], want)


def test_topk_decode_contexts_sampled():
    """Decode: logical positions 0 .. context-1 of 64 sequences x 6 tokens
    with contexts of 4096..65536 positions (most rows beyond the LDS cache)."""
    lens = workloads.decode_lengths()
    Q = workloads.WORKLOADS["decode"].extra["q_per_seq"]
    T = lens.shape[0] * Q
    ctx = np.array([lens[t // Q] - Q + (t % Q) + 1 for t in range(T)])
    C = int(lens.max())
    scores = workloads.index_scores(T, C, seed=51, kind="normal", device="cuda")
    ks, ke = _i32(np.zeros(T)), _i32(ctx)
    got = run(scores, ks, ke, 2048)
    rows = np.arange(0, T, 7)
    want = topk_indices_ref(scores.cpu().numpy()[rows], ks.numpy()[rows], ke.numpy()[rows], 2048)
    assert np.array_equal(got[rows], want)


def test_topk_then_forward_chain():
    """Scores -> top-k -> sparse forward on the GPU, against the top-k oracle
    followed by the forward oracle (packed documents, 8 heads, topk 256)."""
    d = workloads.make_flat("varlen16k", num_tokens=1500, num_heads=8, topk=256, seed=9)
    T = 1500
    ks, ke = workloads.causal_ranges(d["cu_seqlens"].numpy(), T)
    scores = workloads.index_scores(T, T, seed=61, kind="normal")
    dsa = _dsa()
    idx = dsa.topk_indices(scores.to(DEV), ks.to(DEV), ke.to(DEV), 256)
    out, lse = dsa.sparse_mla_fwd(d["q"].to(DEV), d["kv"].to(DEV), idx, d["sm_scale"])
    torch.cuda.synchronize()
    ridx = topk_indices_ref(scores.numpy(), ks.numpy(), ke.numpy(), 256)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ro, rl = sparse_mla_fwd_ref(d["q"].float().numpy(), d["kv"].float().numpy(), ridx, d["sm_scale"])
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.abs(o - ro) <= 2e-2 + 2e-2 * np.abs(ro))
    assert np.all(np.abs(l - rl) <= 1e-3 + 1e-3 * np.abs(rl))
