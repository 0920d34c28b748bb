"""GPU parity of the HIP sparse MLA forward against the CPU oracle.

Every case calls the library through the C ABI (dsa_sparse_mla_amd binding)
and compares element by element with oracle/ on the same seeded inputs.

Tolerance: O within atol = rtol = 2e-2 (the tolerance both kernels met in
"feat: add XTuner TileLang sparse MLA backend", Performance > Isolated sparse
MLA forward) and LSE within atol = rtol = 1e-3. Row with no key: O exactly 0
and LSE exactly -inf. Where the result is exact by construction (a single
key; the same key list reached two ways) the check is bitwise.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import map_paged_indices, sparse_mla_fwd_paged_ref, sparse_mla_fwd_ref

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3
DEV = "cuda"


def _dsa():
    import dsa_sparse_mla_amd as dsa
    return dsa


def np32(t):
    return t.detach().float().cpu().numpy()


def check(o, l, ro, rl, label=""):
    o = np.asarray(o, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(l), empty), f"{label}: -inf LSE pattern differs"
    assert np.all(o[empty] == 0), f"{label}: O of an empty row is not 0"
    full = ~empty
    if full.any():
        do = np.abs(o[full] - ro[full])
        dl = np.abs(l[full] - rl[full])
        bad_o = do > O_TOL + O_TOL * np.abs(ro[full])
        bad_l = dl > LSE_TOL + LSE_TOL * np.abs(rl[full])
        rel = np.linalg.norm(o[full] - ro[full]) / max(np.linalg.norm(ro[full]), 1e-30)
        print(f"[{label}] max|dO|={do.max():.3e} rel_fro={rel:.3e} max|dLSE|={dl.max():.3e}")
        assert not bad_o.any(), f"{label}: {bad_o.sum()} O elements outside tolerance, max {do.max()}"
        assert not bad_l.any(), f"{label}: {bad_l.sum()} LSE elements outside tolerance, max {dl.max()}"
        assert rel < 1e-2, f"{label}: relative Frobenius error {rel}"
    assert np.isfinite(o).all()


def run_flat(q, kv, idx, sm, **kw):
    out, lse = _dsa().sparse_mla_fwd(q.to(DEV), kv.to(DEV), idx.to(DEV), sm, **kw)
    torch.cuda.synchronize()
    return out, lse


def ref_flat(q, kv, idx, sm, tokens=None):
    if tokens is not None:
        q, idx = q[tokens], idx[tokens]
    return sparse_mla_fwd_ref(np32(q), np32(kv), idx.cpu().numpy(), sm)


def random_case(T, H, N, topk, seed, pad_frac=0.3, junk=True):
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((N, 576), generator=g).to(torch.bfloat16)
    idx = rng.integers(0, N, size=(T, topk)).astype(np.int32)
    mask = rng.random((T, topk)) < pad_frac
    idx[mask] = -1
    if junk:
        j = rng.random((T, topk)) < 0.05
        idx[j] = rng.choice(np.array([N, N + 7, -2, -(2 ** 31), 2 ** 31 - 1], dtype=np.int64),
                            size=int(j.sum())).astype(np.int32)
    return q, kv, torch.from_numpy(idx)


# ------------------------------------------------------------------ workloads, small

def test_short_prefill_full():
    d = workloads.make_flat("short")
    out, lse = run_flat(d["q"], d["kv"], d["indices"], d["sm_scale"])
    check(np32(out), np32(lse), *ref_flat(d["q"], d["kv"], d["indices"], d["sm_scale"]), "short")


def test_swe_prefill_small():
    d = workloads.make_flat("swe", num_tokens=300)
    out, lse = run_flat(d["q"], d["kv"], d["indices"], d["sm_scale"])
    check(np32(out), np32(lse), *ref_flat(d["q"], d["kv"], d["indices"], d["sm_scale"]), "swe300")


def test_wide_prefill_small():
    d = workloads.make_flat("wide", num_tokens=200, topk=2048)
    out, lse = run_flat(d["q"], d["kv"], d["indices"], d["sm_scale"])
    check(np32(out), np32(lse), *ref_flat(d["q"], d["kv"], d["indices"], d["sm_scale"]), "wide200")


def test_varlen_small_and_document_isolation():
    d = workloads.make_flat("varlen16k", num_tokens=9000, num_heads=16, topk=512)
    out, lse = run_flat(d["q"], d["kv"], d["indices"], d["sm_scale"], num_splits=1)
    toks = np.arange(0, 9000, 11)
    check(np32(out)[toks], np32(lse)[toks],
          *ref_flat(d["q"], d["kv"], d["indices"], d["sm_scale"], toks), "varlen9000")
    cu = d["cu_seqlens"].numpy()
    assert len(cu) >= 4                          # documents are at most 4096 long
    a, b = int(cu[1]), int(cu[2])            # the second document
    kv2 = d["kv"].clone()
    kv2[:a] = torch.randn_like(kv2[:a].float()).to(torch.bfloat16)
    kv2[b:] = 0
    out2, lse2 = run_flat(d["q"], kv2, d["indices"], d["sm_scale"], num_splits=1)
    assert torch.equal(out2[a:b], out[a:b]) and torch.equal(lse2[a:b], lse[a:b])


def test_paged_decode_small():
    d = workloads.make_paged(num_seqs=6, q_per_seq=6, min_len=1000, max_len=5000, topk=2048)
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    out, lse = _dsa().sparse_mla_fwd_paged(dev["q"], dev["kv_pages"], dev["page_table"],
                                           dev["seq_lens"], dev["indices"], d["sm_scale"],
                                           d["q_per_seq"])
    torch.cuda.synchronize()
    ro, rl = sparse_mla_fwd_paged_ref(np32(d["q"]), np32(d["kv_pages"]), d["page_table"].numpy(),
                                      d["seq_lens"].numpy(), d["indices"].numpy(), d["sm_scale"],
                                      d["q_per_seq"])
    check(np32(out), np32(lse), ro, rl, "paged36")


# ------------------------------------------------------------------ shapes and edge cases

@pytest.mark.parametrize("H", [1, 3, 8, 15, 16, 17, 31, 32, 33, 48, 64, 65, 100, 128])
def test_head_counts(H):
    q, kv, idx = random_case(T=24, H=H, N=900, topk=300, seed=H)
    out, lse = run_flat(q, kv, idx, 0.05)
    check(np32(out), np32(lse), *ref_flat(q, kv, idx, 0.05), f"H={H}")


@pytest.mark.parametrize("topk", [1, 2, 15, 16, 17, 63, 64, 65, 129, 2047, 2048, 2049, 4500])
def test_topk_and_ragged_tails(topk):
    q, kv, idx = random_case(T=10, H=8, N=5000, topk=topk, seed=topk, pad_frac=0.1)
    out, lse = run_flat(q, kv, idx, 1 / 24)
    check(np32(out), np32(lse), *ref_flat(q, kv, idx, 1 / 24), f"topk={topk}")


@pytest.mark.parametrize("H", [8, 64])
@pytest.mark.parametrize("splits", [2, 3, 7, 16])
def test_forced_splits(H, splits):
    q, kv, idx = random_case(T=9, H=H, N=3000, topk=2048, seed=100 + splits, pad_frac=0.5)
    idx[3] = -1                                  # an empty row
    idx[4, 100:] = -1                            # later splits of this row are empty
    out, lse = run_flat(q, kv, idx, 1 / 24, num_splits=splits)
    check(np32(out), np32(lse), *ref_flat(q, kv, idx, 1 / 24), f"H={H} splits={splits}")


def test_empty_rows():
    q, kv, idx = random_case(T=20, H=8, N=100, topk=64, seed=7, junk=False)
    idx[::3] = -1
    idx[1, :] = 100                              # all out of range
    out, lse = run_flat(q, kv, idx, 0.05)
    ro, rl = ref_flat(q, kv, idx, 0.05)
    check(np32(out), np32(lse), ro, rl, "empty")
    assert torch.isneginf(lse[::3]).all() and (out[::3] == 0).all()


def test_single_key_is_exact():
    q, kv, _ = random_case(T=16, H=8, N=50, topk=1, seed=9)
    keys = torch.randint(0, 50, (16,), generator=torch.Generator().manual_seed(3))
    idx = torch.full((16, 300), -1, dtype=torch.int32)
    idx[torch.arange(16), torch.randint(0, 300, (16,))] = keys.int()
    for splits in (1, 3):
        out, lse = run_flat(q, kv, idx, 0.05, num_splits=splits)
        want = kv[keys.long(), :512].unsqueeze(1).expand(16, 8, 512)
        assert torch.equal(out.cpu(), want), f"splits={splits}"
        ro, rl = ref_flat(q, kv, idx, 0.05)
        check(np32(out), np32(lse), ro, rl, f"single-key splits={splits}")


def test_duplicate_indices_count_twice():
    q, kv, _ = random_case(T=4, H=8, N=40, topk=8, seed=11)
    idx = torch.tensor([[3, 3, 5, -1], [7, 7, 7, 7], [1, 2, 3, 4], [9, 9, -1, 2]], dtype=torch.int32)
    out, lse = run_flat(q, kv, idx, 0.05)
    check(np32(out), np32(lse), *ref_flat(q, kv, idx, 0.05), "duplicates")


@pytest.mark.parametrize("H", [8, 64])
def test_peaky_scores_stay_finite(H):
    q, kv, idx = random_case(T=32, H=H, N=2000, topk=512, seed=12, junk=False)
    q = (q.float() * 30).to(torch.bfloat16)
    out, lse = run_flat(q, kv, idx, 1 / 24)
    assert torch.isfinite(out.float()).all()
    check(np32(out), np32(lse), *ref_flat(q, kv, idx, 1 / 24), f"peaky H={H}")


@pytest.mark.parametrize("H", [16, 64])
@pytest.mark.parametrize("sm", [0.0, 1e-4, 0.5])
def test_softmax_scale_range(sm, H):
    """sm_scale = 0 gives uniform weights (O = mean of the latent rows, LSE =
    log of the key count); a large scale makes every row nearly one-hot."""
    q, kv, idx = random_case(T=40, H=H, N=3000, topk=700, seed=13)
    out, lse = run_flat(q, kv, idx, sm)
    ro, rl = ref_flat(q, kv, idx, sm)
    check(np32(out), np32(lse), ro, rl, f"scale{sm} H={H}")
    if sm == 0.0:
        n = ((idx >= 0) & (idx < 3000)).sum(1).numpy()
        np.testing.assert_allclose(np32(lse), np.log(n)[:, None].repeat(H, 1), rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("H", [8, 64])
@pytest.mark.parametrize("splits", [1, 3])
def test_rising_scores_move_the_reference(H, splits):
    """Scores that climb along the key list (key j at about 200 * j / topk,
    natural-log units) force the running maximum to move many times inside a
    row, by more than any lazy-rescale slack, so every rescale path of O and
    of the row sum runs; per row the first keys then weigh ~e^-200."""
    T, N, topk = 12, 2048, 1500
    g = torch.Generator().manual_seed(21)
    u = torch.randn(576, generator=g)
    q = (u[None, None, :] + 0.3 * torch.randn((T, H, 576), generator=g)).to(torch.bfloat16)
    ramp = torch.arange(N, dtype=torch.float32) / topk
    kv = (8.3 * ramp[:, None] * u[None, :] + 0.5 * torch.randn((N, 576), generator=g)).to(torch.bfloat16)
    idx = torch.arange(topk, dtype=torch.int32).repeat(T, 1)
    idx[1::2] = torch.flip(idx[1::2], dims=[1])   # falling order too: the maximum comes first
    out, lse = run_flat(q, kv, idx, 1 / 24, num_splits=splits)
    check(np32(out), np32(lse), *ref_flat(q, kv, idx, 1 / 24), f"rising H={H} splits={splits}")


def test_paged_wide_heads():
    """The 64-head kernel on the paged cache (page mapping fused in the index stage)."""
    d = workloads.make_paged(num_seqs=3, q_per_seq=4, num_heads=64, min_len=1500, max_len=4000, topk=1024)
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    out, lse = _dsa().sparse_mla_fwd_paged(dev["q"], dev["kv_pages"], dev["page_table"],
                                           dev["seq_lens"], dev["indices"], d["sm_scale"],
                                           d["q_per_seq"])
    torch.cuda.synchronize()
    ro, rl = sparse_mla_fwd_paged_ref(np32(d["q"]), np32(d["kv_pages"]), d["page_table"].numpy(),
                                      d["seq_lens"].numpy(), d["indices"].numpy(), d["sm_scale"],
                                      d["q_per_seq"])
    check(np32(out), np32(lse), ro, rl, "paged H=64")


@pytest.mark.parametrize("H,T,splits", [(64, 3000, 1), (128, 1500, 1), (64, 1500, 2)])
def test_many_mixed_rows(H, T, splits):
    """About 3000 (token, split, head block) workgroups of the 64-head kernel
    (several per CU, so later ones start while others run) with row lengths
    from 0 to 8 tiles shuffled among -1 and junk values: empty rows, rows of
    1-3 tiles and longer ones side by side. Repeated runs are bitwise equal."""
    N, topk = 4096, 256
    g = torch.Generator().manual_seed(40 + H + splits)
    rng = np.random.default_rng(40 + H + splits)
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((N, 576), generator=g).to(torch.bfloat16)
    idx = np.full((T, topk), -1, dtype=np.int32)
    nvalid = rng.integers(0, topk + 1, size=T)
    nvalid[rng.random(T) < 0.05] = 0
    for t in range(T):
        row = idx[t]
        row[:nvalid[t]] = rng.integers(0, N, size=nvalid[t])
        row[nvalid[t]:] = rng.choice(np.array([-1, -1, -1, N, -5], dtype=np.int32), size=topk - nvalid[t])
        rng.shuffle(row)
    idx = torch.from_numpy(idx)
    out, lse = run_flat(q, kv, idx, 1 / 24, num_splits=splits)
    check(np32(out), np32(lse), *ref_flat(q, kv, idx, 1 / 24), f"mixed H={H} T={T} splits={splits}")
    out2, lse2 = run_flat(q, kv, idx, 1 / 24, num_splits=splits)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_paged_many_mixed_rows():
    """The paged 64-head kernel over 1800 query tokens of 300 short sequences
    (contexts of 40-700 tokens, so many rows hold fewer than topk entries)."""
    d = workloads.make_paged(num_seqs=300, q_per_seq=6, num_heads=64, min_len=40, max_len=700, topk=128)
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    out, lse = _dsa().sparse_mla_fwd_paged(dev["q"], dev["kv_pages"], dev["page_table"],
                                           dev["seq_lens"], dev["indices"], d["sm_scale"],
                                           d["q_per_seq"])
    torch.cuda.synchronize()
    ro, rl = sparse_mla_fwd_paged_ref(np32(d["q"]), np32(d["kv_pages"]), d["page_table"].numpy(),
                                      d["seq_lens"].numpy(), d["indices"].numpy(), d["sm_scale"],
                                      d["q_per_seq"])
    check(np32(out), np32(lse), ro, rl, "paged mixed H=64")


def test_strided_inputs_and_outputs():
    T, H, N, k = 12, 8, 700, 200
    q_big, kv, idx = random_case(T=T, H=H * 2, N=N, topk=k, seed=13)
    q = q_big[:, ::2]                            # oracle input
    kv_big = torch.zeros((N, 640), dtype=torch.bfloat16)
    kv_big[:, :576] = kv                         # row stride 640
    idx_big = torch.full((T, k + 16), -1, dtype=torch.int32)
    idx_big[:, :k] = idx
    qd = q_big.to(DEV)[:, ::2]                   # head stride 2*576 on the device
    assert qd.stride(1) == 2 * 576
    out_big = torch.full((T, H, 2 * 512), 7.0, dtype=torch.bfloat16, device=DEV)
    lse_big = torch.full((T, 2 * H), 7.0, dtype=torch.float32, device=DEV)
    out = out_big[:, :, :512]
    lse = lse_big[:, :H]
    _dsa().sparse_mla_fwd(qd, kv_big.to(DEV)[:, :576], idx_big.to(DEV)[:, :k], 0.05, out=out, lse=lse)
    torch.cuda.synchronize()
    check(np32(out), np32(lse), *ref_flat(q, kv, idx, 0.05), "strided")
    assert (out_big[:, :, 512:] == 7.0).all() and (lse_big[:, H:] == 7.0).all()


# ------------------------------------------------------------------ bitwise properties

def test_deterministic_and_padding_invariant():
    d = workloads.make_flat("swe", num_tokens=400)
    a = run_flat(d["q"], d["kv"], d["indices"], d["sm_scale"], num_splits=1)
    b = run_flat(d["q"], d["kv"], d["indices"], d["sm_scale"], num_splits=1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    idx = d["indices"].numpy()
    rng = np.random.default_rng(0)
    wide = np.full((idx.shape[0], idx.shape[1] + 1), -1, dtype=np.int32)   # 2049 entries
    for t in range(idx.shape[0]):
        row = idx[t][idx[t] >= 0]
        pos = np.sort(rng.choice(wide.shape[1], len(row), replace=False))
        wide[t, pos] = row                       # same keys, same order, -1 elsewhere
    c = run_flat(d["q"], d["kv"], torch.from_numpy(wide), d["sm_scale"], num_splits=2)
    e = run_flat(d["q"], d["kv"], torch.from_numpy(wide), d["sm_scale"], num_splits=2)
    assert torch.equal(c[0], e[0]) and torch.equal(c[1], e[1])
    check(np32(c[0]), np32(c[1]), np32(a[0]), np32(a[1]), "2049-wide vs 2048")


def test_paged_equals_flat_bitwise_and_page_permutation():
    d = workloads.make_paged(num_seqs=5, q_per_seq=6, min_len=3000, max_len=9000, topk=2048)
    P, ps, _ = d["kv_pages"].shape
    dsa = _dsa()
    dv = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    out_p, lse_p = dsa.sparse_mla_fwd_paged(dv["q"], dv["kv_pages"], dv["page_table"], dv["seq_lens"],
                                            dv["indices"], d["sm_scale"], 6, num_splits=1)
    phys = map_paged_indices(d["indices"].numpy(), d["page_table"].numpy(), d["seq_lens"].numpy(),
                             P, ps, 6).astype(np.int32)
    out_f, lse_f = dsa.sparse_mla_fwd(dv["q"], dv["kv_pages"].reshape(P * ps, 576),
                                      torch.from_numpy(phys).to(DEV), d["sm_scale"], num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_f) and torch.equal(lse_p, lse_f)
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(1))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P)
    pages2 = torch.empty_like(dv["kv_pages"])
    pages2[inv.to(DEV)] = dv["kv_pages"]         # page p moves to slot inv[p]
    table = d["page_table"].clone()
    m = table >= 0
    table[m] = inv[table[m].long()].int()
    out_q, lse_q = dsa.sparse_mla_fwd_paged(dv["q"], pages2, table.to(DEV), dv["seq_lens"],
                                            dv["indices"], d["sm_scale"], 6, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(out_q, out_p) and torch.equal(lse_q, lse_p)


def test_paged_masking_edges():
    """Positions past seq_len, unmapped table slots and bad page ids are skipped."""
    d = workloads.make_paged(num_seqs=3, q_per_seq=2, min_len=300, max_len=700, topk=256)
    idx = d["indices"].clone()
    idx[0, :20] = 10 ** 6                         # past every sequence
    idx[1, :5] = -3
    table = d["page_table"].clone()
    table[2, 0] = -1                              # unmapped page
    table[2, 1] = d["kv_pages"].shape[0] + 5      # page id past the cache
    idx[2, :] = -1                                # sequence 1, query 0: all skipped
    dv = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    out, lse = _dsa().sparse_mla_fwd_paged(dv["q"], dv["kv_pages"], table.to(DEV), dv["seq_lens"],
                                           idx.to(DEV), d["sm_scale"], 2)
    torch.cuda.synchronize()
    ro, rl = sparse_mla_fwd_paged_ref(np32(d["q"]), np32(d["kv_pages"]), table.numpy(),
                                      d["seq_lens"].numpy(), idx.numpy(), d["sm_scale"], 2)
    check(np32(out), np32(lse), ro, rl, "paged-edges")


# ------------------------------------------------------------------ full sizes, sampled

def _sample(T, n, seed=0):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, n, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


@pytest.mark.parametrize("name,nsample", [("swe", 256), ("wide", 48), ("varlen16k", 40),
                                          ("varlen32k", 32)])
def test_full_size_sampled(name, nsample):
    dev = "cuda" if name != "swe" else "cpu"
    d = workloads.make_flat(name, device=dev)
    out, lse = run_flat(d["q"], d["kv"], d["indices"], d["sm_scale"])
    toks = _sample(d["q"].shape[0], nsample)
    tt = torch.from_numpy(toks).to(d["q"].device)
    q_s = d["q"][tt].cpu()
    idx_s = d["indices"][tt].cpu()
    ro, rl = sparse_mla_fwd_ref(np32(q_s), np32(d["kv"]), idx_s.numpy(), d["sm_scale"])
    check(np32(out)[toks], np32(lse)[toks], ro, rl, f"{name} full, {len(toks)} sampled tokens")


def test_decode_full_size_all_sequences():
    """The decode workload at full size (64 sequences x 6 tokens, contexts up
    to 65536, paged bf16 cache), in the launch configuration bench.py times;
    every token against the oracle. The oracle takes eight sequences at a
    time with only their pages (compacted and renumbered), which bounds its
    memory."""
    d = workloads.make_paged(device="cuda")
    dsa = _dsa()
    out, lse = dsa.sparse_mla_fwd_paged(d["q"], d["kv_pages"], d["page_table"], d["seq_lens"],
                                        d["indices"], d["sm_scale"], d["q_per_seq"])
    torch.cuda.synchronize()
    Q = d["q_per_seq"]
    S = d["page_table"].shape[0]
    table_all = d["page_table"].cpu().numpy()
    lens_all = d["seq_lens"].cpu().numpy()
    o_all, l_all = np32(out), np32(lse)
    for s0 in range(0, S, 8):
        seqs = np.arange(s0, min(S, s0 + 8))
        toks = (seqs[:, None] * Q + np.arange(Q)).ravel()
        table = table_all[seqs]
        used = np.unique(table[table >= 0])
        remap = np.full(d["kv_pages"].shape[0], -1, dtype=np.int64)
        remap[used] = np.arange(used.size)
        small = np.where(table >= 0, remap[np.maximum(table, 0)], -1).astype(np.int32)
        pages = np32(d["kv_pages"][torch.from_numpy(used).to(DEV)])
        tt = torch.from_numpy(toks).to(DEV)
        ro, rl = sparse_mla_fwd_paged_ref(np32(d["q"][tt]), pages, small, lens_all[seqs],
                                          d["indices"][tt].cpu().numpy(), d["sm_scale"], Q)
        check(o_all[toks], l_all[toks], ro, rl, f"decode full, sequences {s0}..{seqs[-1]}")