"""The entry points under HIP graph capture ("feat: add XTuner TileLang
sparse MLA backend", Validation: the serving runs use CUDA graphs).

Each call only enqueues kernels on the caller's stream (no allocation, no
synchronisation, no memset node), so it can be captured. The test captures
one call with preallocated outputs, replays the graph several times with
eager work on the same buffers between the replays, and requires every
replay to equal the eager result bit for bit (and the eager result to match
the oracle at the forward's tolerance); the backward's atomically summed
outputs are held to a bound instead (see its test).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import sparse_mla_bwd_ref, sparse_mla_fwd_paged_ref, sparse_mla_fwd_ref, topk_indices_ref

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dsa():
    import dsa_sparse_mla_amd as dsa
    return dsa


def _replays(fn, outs, reps=3):
    """Eager result, then `reps` graph replays, each after the outputs were
    overwritten by eager work; returns (eager, [replays])."""
    fn()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    got = []
    for r in range(reps):
        for o in outs:
            o.fill_(r + 3)         # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got.append([o.clone() for o in outs])
    return eager, got


@pytest.mark.parametrize("splits", [1, 4])
def test_flat_forward_captured(splits):
    d = workloads.make_flat("swe", num_tokens=300, topk=512, seed=81)
    dsa = _dsa()
    q, kv, idx = d["q"].to(DEV), d["kv"].to(DEV), d["indices"].to(DEV)
    T, H = q.shape[:2]
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    _, nbytes = dsa.workspace_size(T, H, 512, splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)

    def fn():
        dsa.sparse_mla_fwd(q, kv, idx, d["sm_scale"], out=out, lse=lse, num_splits=splits, workspace=ws)

    eager, got = _replays(fn, [out, lse])
    for rep in got:
        assert torch.equal(rep[0], eager[0]) and torch.equal(rep[1], eager[1])
    ro, rl = sparse_mla_fwd_ref(d["q"].float().numpy(), d["kv"].float().numpy(), d["indices"].numpy(),
                                d["sm_scale"])
    o = eager[0].float().cpu().numpy()
    assert np.all(np.abs(o - ro) <= 2e-2 + 2e-2 * np.abs(ro))


@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("which", ["paged", "noalloc"])
def test_paged_forward_captured(which, splits):
    d = workloads.make_paged(num_seqs=8, q_per_seq=6, min_len=1000, max_len=6000, topk=2048, seed=82)
    dv = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    dsa = _dsa()
    T, H = dv["q"].shape[:2]
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    got_splits, nbytes = dsa.workspace_size(T, H, 2048, splits)
    assert got_splits == splits
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    args = (dv["q"], dv["kv_pages"], dv["page_table"], dv["seq_lens"], dv["indices"], dv["sm_scale"],
            dv["q_per_seq"])

    def fn():
        if which == "paged":
            dsa.sparse_mla_fwd_paged(*args, out=out, lse=lse, num_splits=splits, workspace=ws)
        else:
            dsa.sparse_mla_fwd_paged_noalloc(*args, out=out, lse=lse, num_splits=splits)

    eager, got = _replays(fn, [out, lse])
    for rep in got:
        assert torch.equal(rep[0], eager[0]) and torch.equal(rep[1], eager[1])
    ro, rl = sparse_mla_fwd_paged_ref(d["q"].float().numpy(), d["kv_pages"].float().numpy(),
                                      d["page_table"].numpy(), d["seq_lens"].numpy(), d["indices"].numpy(),
                                      d["sm_scale"], d["q_per_seq"])
    o = eager[0].float().cpu().numpy()
    assert np.all(np.abs(o - ro) <= 2e-2 + 2e-2 * np.abs(ro))


def test_topk_captured():
    T = 700
    scores = workloads.index_scores(T, T, seed=83, kind="ties").to(DEV)
    ks, ke = workloads.causal_ranges(None, T)
    ks, ke = ks.to(DEV), ke.to(DEV)
    idx = torch.empty((T, 256), dtype=torch.int32, device=DEV)
    dsa = _dsa()

    def fn():
        dsa.topk_indices(scores, ks, ke, 256, indices=idx)

    eager, got = _replays(fn, [idx])
    for rep in got:
        assert torch.equal(rep[0], eager[0])
    want = topk_indices_ref(scores.cpu().numpy(), ks.cpu().numpy(), ke.cpu().numpy(), 256)
    assert np.array_equal(eager[0].cpu().numpy(), want)


@pytest.mark.parametrize("H", [8, 64])
def test_backward_captured(H):
    """The backward under capture (8 heads: the kv-major schedule; 64: the
    split one). Between replays the outputs and the whole workspace are
    overwritten, so every part a call reads (masks, ranks, P and s*dS, the
    dkv pass's work-queue counters) must be rebuilt inside the captured call.
    The split schedule's dq is written by one workgroup per token and must
    equal the eager result bit for bit; dkv (and the kv-major dq) are sums
    of atomic adds whose order may change from call to call, so they must
    agree to 1e-5 of the tensor's largest magnitude. The eager result is
    checked against the oracle (Frobenius error within 1e-2, the backward
    tests' end-to-end bound: out and LSE come from the library's forward)."""
    dsa = _dsa()
    T, N, topk, sm = 300, 200, 160, 1 / 24
    rng = np.random.default_rng(83 + H)
    g = torch.Generator().manual_seed(83 + H)
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((N, 576), generator=g).to(torch.bfloat16)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    idx = np.stack([rng.permutation(N)[:topk] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, topk)) < 0.3] = -1
    qd, kd, idd, dod = q.to(DEV), kv.to(DEV), torch.from_numpy(idx).to(DEV), dout.to(DEV)
    out, lse = dsa.sparse_mla_fwd(qd, kd, idd, sm)
    sched, nbytes = dsa.bwd_workspace_size(T, H, N, topk)
    assert sched == ("kv-major" if H == 8 else "split")
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    dq = torch.empty((T, H, 576), dtype=torch.float32, device=DEV)
    dkv = torch.empty((N, 576), dtype=torch.float32, device=DEV)

    def fn():
        dsa.sparse_mla_bwd(qd, kd, idd, sm, out, lse, dod, dq=dq, dkv=dkv, workspace=ws)

    eager, got = _replays(fn, [dq, dkv, ws])
    for rep in got:
        for i in range(2):
            a, b = rep[i], eager[i]
            if i == 0 and sched == "split":
                assert torch.equal(a, b)
            else:
                assert torch.allclose(a, b, rtol=0.0, atol=1e-5 * float(b.abs().max()))
    rdq, rdkv = sparse_mla_bwd_ref(q.double().numpy(), kv.double().numpy(), idx, sm, dout.double().numpy())
    for x, r in ((eager[0], rdq), (eager[1], rdkv)):
        x = x.double().cpu().numpy()
        assert np.linalg.norm(x - r) <= 1e-2 * np.linalg.norm(r)
