"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each pin is a function of the oracle callable, so that test_oracle_mutants.py
can run the same pins against copies of the oracle with a planted mistake and
check that some pin fails.

Pins (what fixes each part of the method):
  hand-worked fixture  closed forms derived by hand (tests/golden)
  dense causal         full causal index rows reduce the method to dense causal
                       single-KV-head attention: torch's scaled_dot_product_attention
                       in float64 (a library routine); LSE via scipy's logsumexp
  single key           O = that key's V row exactly, LSE = its scaled score
  zero query           LSE = ln |J|, O = mean of the V rows
  brute force          scalar Python loops, no max shift, math.fsum
  permutation          order of the index row does not matter
  padding              -1 and out-of-range entries anywhere change nothing
  heads                permuting query heads permutes O and LSE
  peaky                one dominant key: O -> its V row within exp(-gap) bound
  paged == flat        a cache built by scattering flat rows into random pages
                       gives the flat result exactly; mapping checked by hand
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import DQK, DV, map_paged_indices, sparse_mla_fwd_paged_ref, sparse_mla_fwd_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape, scale=1.0):
    # bf16-representable values, so the same inputs also suit the GPU path
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return x.to(torch.bfloat16).float().numpy()


# ------------------------------------------------------------------ pins

def pin_hand_worked(fwd):
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        case = json.load(f)
    T = len(case["indices"])
    H = case["num_heads"]
    N = case["num_kv"]
    q = np.zeros((T, H, DQK))
    kv = np.zeros((N, DQK))
    for t, h, d, v in case["q_nonzero"]:
        q[t, h, d] = v
    for r, d, v in case["kv_nonzero"]:
        kv[r, d] = v
    out, lse = fwd(q, kv, np.array(case["indices"]), case["sm_scale"])
    env = {"e": math.e, "log": math.log, "exp": math.exp, "inf": math.inf}
    for exp_row in case["expected"]:
        t, h = exp_row["token"], exp_row["head"]
        want_lse = eval(exp_row["lse"], {"__builtins__": {}}, env)  # our own fixture
        if math.isinf(want_lse):
            assert lse[t, h] == want_lse
        else:
            assert abs(lse[t, h] - want_lse) < 1e-12, (t, h, lse[t, h], want_lse)
        want_o = np.zeros(DV)
        for c, expr in exp_row["o"].items():
            want_o[int(c)] = eval(expr, {"__builtins__": {}}, env)
        np.testing.assert_allclose(out[t, h], want_o, rtol=0, atol=1e-12)


def pin_dense_causal(fwd, T=40, H=3, seed=0):
    """Rows holding every causal key 0..t equal dense causal attention."""
    rng = np.random.default_rng(seed)
    q = _rand(rng, T, H, DQK)
    kv = _rand(rng, T, DQK)
    sm = 1.0 / 24.0
    idx = np.full((T, T + 5), -1, dtype=np.int64)
    for t in range(T):
        idx[t, : t + 1] = rng.permutation(t + 1)
    out, lse = fwd(q, kv, idx, sm)
    # library routine: dense causal attention, one KV head shared by all H
    qt = torch.from_numpy(q).double().permute(1, 0, 2)[None]            # [1,H,T,576]
    k = torch.from_numpy(kv).double()[None, None].expand(1, H, T, DQK)
    v = torch.from_numpy(kv[:, :DV]).double()[None, None].expand(1, H, T, DV)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, k, v, is_causal=True, scale=sm)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    scores = np.einsum("thd,sd->ths", q.astype(np.float64), kv.astype(np.float64)) * sm
    mask = np.tril(np.ones((T, T), dtype=bool))[:, None, :]
    ref_lse = logsumexp(np.where(mask, scores, -np.inf), axis=-1)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def pin_single_key(fwd, seed=1):
    """J = {i}: O is V row i exactly and LSE is the scaled score."""
    rng = np.random.default_rng(seed)
    T, H, N = 5, 4, 9
    q = _rand(rng, T, H, DQK)
    kv = _rand(rng, N, DQK)
    sm = 0.0625
    keys = rng.integers(0, N, size=T)
    idx = np.full((T, 6), -1, dtype=np.int64)
    idx[np.arange(T), rng.integers(0, 6, size=T)] = keys
    out, lse = fwd(q, kv, idx, sm)
    for t in range(T):
        for h in range(H):
            assert np.array_equal(out[t, h], kv[keys[t], :DV].astype(np.float64))
            want = sm * math.fsum(float(a) * float(b) for a, b in zip(q[t, h], kv[keys[t]]))
            assert abs(lse[t, h] - want) < 1e-12 * max(1.0, abs(want))


def pin_zero_query(fwd, seed=2):
    """q = 0: every score is 0, so LSE = ln |J| and O is the mean of the V rows."""
    rng = np.random.default_rng(seed)
    N = 30
    kv = _rand(rng, N, DQK)
    rows = [rng.choice(N, n, replace=False) for n in (1, 7, 30)]
    idx = np.full((3, 32), -1, dtype=np.int64)
    for t, r in enumerate(rows):
        idx[t, : len(r)] = r
    q = np.zeros((3, 2, DQK))
    out, lse = fwd(q, kv, idx, 0.3)
    for t, r in enumerate(rows):
        np.testing.assert_allclose(lse[t], np.log(len(r)), rtol=0, atol=1e-14)
        mean = kv[r, :DV].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[t], np.broadcast_to(mean, (2, DV)), rtol=0, atol=1e-14)


def _brute(q, kv, idx, sm):
    T, H, _ = q.shape
    N = kv.shape[0]
    out = np.zeros((T, H, DV))
    lse = np.full((T, H), -math.inf)
    for t in range(T):
        keys = [int(i) for i in idx[t] if 0 <= int(i) < N]
        for h in range(H):
            if not keys:
                continue
            w = [math.exp(sm * math.fsum(float(a) * float(b) for a, b in zip(q[t, h], kv[j])))
                 for j in keys]
            z = math.fsum(w)
            lse[t, h] = math.log(z)
            for c in range(DV):
                out[t, h, c] = math.fsum(wj * float(kv[j, c]) for wj, j in zip(w, keys)) / z
    return out, lse


def pin_brute_force(fwd, seed=3):
    """Tiny inputs against scalar loops with no max shift (a second formulation)."""
    rng = np.random.default_rng(seed)
    T, H, N, k = 4, 3, 16, 8
    q = _rand(rng, T, H, DQK, scale=0.5)
    kv = _rand(rng, N, DQK)
    idx = rng.integers(-3, N + 3, size=(T, k))
    idx[3] = -1  # one empty row
    sm = 1.0 / 24.0
    out, lse = fwd(q, kv, idx, sm)
    bo, bl = _brute(q, kv, idx, sm)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-13)


def pin_permutation_and_padding(fwd, seed=4):
    """Row order, -1 padding anywhere and out-of-range entries change nothing."""
    rng = np.random.default_rng(seed)
    T, H, N = 6, 2, 50
    q = _rand(rng, T, H, DQK)
    kv = _rand(rng, N, DQK)
    sm = 1.0 / 24.0
    base = np.stack([rng.choice(N, 20, replace=False) for _ in range(T)])
    o0, l0 = fwd(q, kv, base, sm)
    perm = np.stack([rng.permutation(r) for r in base])
    o1, l1 = fwd(q, kv, perm, sm)
    np.testing.assert_allclose(o1, o0, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l0, rtol=1e-13, atol=1e-15)
    junk = np.array([-1, -7, N, N + 100, -(2 ** 31)])
    padded = np.concatenate([base, rng.choice(junk, size=(T, 13))], axis=1)
    padded = np.stack([rng.permutation(r) for r in padded])
    o2, l2 = fwd(q, kv, padded, sm)
    np.testing.assert_allclose(o2, o0, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l2, l0, rtol=1e-13, atol=1e-15)


def pin_heads(fwd, seed=5):
    """Permuting query heads permutes O and LSE."""
    rng = np.random.default_rng(seed)
    T, H, N = 3, 5, 20
    q = _rand(rng, T, H, DQK)
    kv = _rand(rng, N, DQK)
    idx = np.stack([rng.choice(N, 12, replace=False) for _ in range(T)])
    o, l = fwd(q, kv, idx, 0.05)
    p = rng.permutation(H)
    op, lp = fwd(q[:, p], kv, idx, 0.05)
    np.testing.assert_allclose(op, o[:, p], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lp, l[:, p], rtol=1e-13, atol=1e-15)


def pin_peaky(fwd, seed=6):
    """One key ahead by a gap g: |O - V_top| <= (n-1) e^-g (|V_top| + max|V|)."""
    rng = np.random.default_rng(seed)
    N = 40
    kv = _rand(rng, N, DQK)
    q = 30.0 * _rand(rng, 1, 1, DQK)
    sm = 1.0 / 24.0
    idx = np.arange(N)[None]
    out, lse = fwd(q, kv, idx, sm)
    s = sm * (kv.astype(np.float64) @ q[0, 0].astype(np.float64))
    top = int(np.argmax(s))
    gap = s[top] - np.max(np.delete(s, top))
    assert gap > 3.0, gap  # the draw above is peaky enough for the bound to bite
    bound = (N - 1) * math.exp(-gap) * 2 * np.abs(kv[:, :DV]).max()
    assert np.abs(out[0, 0] - kv[top, :DV]).max() <= bound
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert abs(lse[0, 0] - s[top]) <= (N - 1) * math.exp(-gap)


def pin_paged_equals_flat(fwd, fwd_paged, seed=7):
    """A paged cache made by scattering flat rows gives the flat result exactly."""
    rng = np.random.default_rng(seed)
    B, Qps, H, ps, k = 3, 2, 2, 4, 10
    lens = np.array([9, 13, 4])
    npages = -(-lens // ps)
    P = int(npages.sum()) + 2                      # two spare pages
    perm = rng.permutation(P)
    table = np.full((B, 5), -1, dtype=np.int64)
    kv_pages = _rand(rng, P, ps, DQK)
    off = 0
    flat_rows = []                                 # per sequence: flat row of position p
    kv_flat_list = []
    for b in range(B):
        table[b, : npages[b]] = perm[off: off + npages[b]]
        off += npages[b]
        rows = []
        for p in range(lens[b]):
            rows.append(len(kv_flat_list))
            kv_flat_list.append(kv_pages[table[b, p // ps], p % ps])
        flat_rows.append(rows)
    kv_flat = np.stack(kv_flat_list)
    T = B * Qps
    q = _rand(rng, T, H, DQK)
    logical = rng.integers(-2, 16, size=(T, k))
    flat_idx = np.full((T, k), -1)
    for t in range(T):
        b = t // Qps
        for j in range(k):
            p = logical[t, j]
            if 0 <= p < lens[b]:
                flat_idx[t, j] = flat_rows[b][p]
    o_p, l_p = fwd_paged(q, kv_pages, table, lens, logical, 0.05, Qps)
    o_f, l_f = fwd(q, kv_flat, flat_idx, 0.05)
    np.testing.assert_array_equal(o_p, o_f)
    np.testing.assert_array_equal(l_p, l_f)


def pin_page_mapping_by_hand(mapper):
    """Page size 4; sequence 0 owns pages [5, 2], sequence 1 owns [0] (len 3)."""
    table = np.array([[5, 2, -1], [0, -1, -1]])
    lens = np.array([6, 3])
    idx = np.array([[0, 3, 4, 5, 6, -1, 11],      # seq 0, query 0
                    [2, 1, 0, 3, 8, -4, 5]])      # seq 1, query 0
    got = mapper(idx, table, lens, 6, 4, 1)
    want = np.array([[20, 23, 8, 9, -1, -1, -1],   # 6 and 11 are past len 6
                     [2, 1, 0, -1, -1, -1, -1]])   # 3, 8, 5 past len 3
    np.testing.assert_array_equal(got, want)
    for bad in (6, 9, -3):                          # P = 6: pages 6 and up do not exist
        table_bad = np.array([[5, bad, -1], [0, -1, -1]])
        got = mapper(idx, table_bad, lens, 6, 4, 1)
        assert (got[0, 2:4] == -1).all() and got[0, 0] == 20 and got[0, 1] == 23


# ------------------------------------------------------------------ tests

def test_hand_worked():
    pin_hand_worked(sparse_mla_fwd_ref)


def test_dense_causal():
    pin_dense_causal(sparse_mla_fwd_ref)


def test_single_key():
    pin_single_key(sparse_mla_fwd_ref)


def test_zero_query():
    pin_zero_query(sparse_mla_fwd_ref)


def test_brute_force():
    pin_brute_force(sparse_mla_fwd_ref)


def test_permutation_and_padding():
    pin_permutation_and_padding(sparse_mla_fwd_ref)


def test_heads():
    pin_heads(sparse_mla_fwd_ref)


def test_peaky():
    pin_peaky(sparse_mla_fwd_ref)


def test_paged_equals_flat():
    pin_paged_equals_flat(sparse_mla_fwd_ref, sparse_mla_fwd_paged_ref)


def test_page_mapping_by_hand():
    pin_page_mapping_by_hand(map_paged_indices)


def test_fp32_mode_noise_floor():
    """The fp32 mode stays within the GPU tolerance of fp64 (noise-floor check)."""
    rng = np.random.default_rng(8)
    T, H, N = 16, 8, 300
    q = _rand(rng, T, H, DQK)
    kv = _rand(rng, N, DQK)
    idx = np.stack([rng.choice(N, 256, replace=False) for _ in range(T)])
    o64, l64 = sparse_mla_fwd_ref(q, kv, idx, 1 / 24)
    o32, l32 = sparse_mla_fwd_ref(q, kv, idx, 1 / 24, dtype=np.float32)
    assert o32.dtype == np.float32
    assert np.abs(o32 - o64).max() < 1e-5
    assert np.abs(l32 - l64).max() < 1e-4


@pytest.mark.parametrize("name", ["short", "swe", "varlen16k"])
def test_workload_generator_is_deterministic(name):
    import workloads
    kw = {"num_tokens": 300, "num_heads": 2, "topk": 256} if name != "short" else {}
    a = workloads.make(name, **kw)
    b = workloads.make(name, **kw)
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["kv"], b["kv"])
    assert torch.equal(a["indices"], b["indices"])
    idx = a["indices"].numpy()
    T = idx.shape[0]
    for t in range(T):
        row = idx[t][idx[t] >= 0]
        assert len(np.unique(row)) == len(row)       # distinct keys
        assert (row <= t).all()                      # causal
    if name == "varlen16k":
        cu = a["cu_seqlens"].numpy()
        doc = np.searchsorted(cu, np.arange(T), side="right") - 1
        for t in range(T):
            row = idx[t][idx[t] >= 0]
            assert (row >= cu[doc[t]]).all()         # own document only
            assert len(row) == min(t - cu[doc[t]] + 1, 256)


def test_paged_generator_structure():
    import workloads
    d = workloads.make_paged(num_seqs=4, q_per_seq=3, topk=64, min_len=70, max_len=300)
    table = d["page_table"].numpy()
    lens = d["seq_lens"].numpy()
    P = d["kv_pages"].shape[0]
    used = table[table >= 0]
    assert sorted(used.tolist()) == list(range(P))   # a permutation of all pages
    idx = d["indices"].numpy()
    for t in range(idx.shape[0]):
        b, j = divmod(t, 3)
        row = idx[t][idx[t] >= 0]
        assert len(row) == 64 and len(np.unique(row)) == 64
        assert row.max() <= lens[b] - 3 + j
