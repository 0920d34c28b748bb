"""GPU parity of the HIP sparse MLA backward against the CPU backward oracle.

Every case calls the backward through the C ABI and compares dq and dkv
element by element with oracle/ (fp64, recomputed from q, kv, indices and
dout alone). The parity cases hand the kernel the oracle's forward output
(rounded to bf16, as a forward returns it) and LSE, so that only the
backward's own arithmetic is measured; one end-to-end case feeds it the
library's own forward instead, as a training step does.

Tolerance. The pages fix none for the backward; this one follows from the
arithmetic. The kernel rounds sm_scale*dS (and P) to bf16, unit roundoff
2^-8, before its MFMA products; every other operand is an exact bf16 input
and sums are fp32. A CPU emulation of exactly that rounding on the SWE-like
workload gives a relative Frobenius error of 1.6e-3 for dq, and no element
of dq beyond 0.014 * (|ref| + rms of the token's dq). The bound here is
twice that, 3e-2 * (|ref| + rms of the token's row of the result: dq over
its heads and columns, dkv over its 576 columns), plus the Frobenius bound
1e-2. Both add an absolute 1e-4 per element: dS = P (dP - D) subtracts two
fp32 dot products of 512 terms (magnitude ~20, rounding ~1e-6 each), and
where they cancel exactly (one key: P = 1, D = dP) the reference is 0 while
the kernel keeps that residue. End to end, D = dout . out also carries the
forward's own rounding (its O is within the forward's 2e-2 tolerance), an
error common to every key of a token; that case keeps the Frobenius bound
and checks elements only against gross error (1e-1).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import sparse_mla_bwd_ref, sparse_mla_fwd_ref

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dsa():
    import dsa_sparse_mla_amd as dsa
    return dsa


def np64(t):
    return t.detach().double().cpu().numpy()


def check_grad(x, ref, label, elem_tol=3e-2):
    x = np.asarray(x, dtype=np.float64)
    assert np.isfinite(x).all(), f"{label}: non-finite values"
    # scale per first-axis row (one token's dq, one kv row's dkv): rows
    # differ in magnitude (tokens with few keys have larger gradients)
    rows = ref.reshape(ref.shape[0], -1)
    rms_row = np.sqrt(np.mean(rows ** 2, axis=1, keepdims=True))
    rms = float(np.sqrt(np.mean(rows ** 2)))
    err = np.abs(x - ref).reshape(rows.shape)
    bad = err > elem_tol * (np.abs(rows) + rms_row) + 1e-4
    fro, rfro = np.linalg.norm(x - ref), np.linalg.norm(ref)
    print(f"[{label}] max|d|={err.max():.3e} rms(ref)={rms:.3e} rel_fro={fro / max(rfro, 1e-30):.3e}")
    assert not bad.any(), f"{label}: {bad.sum()} elements outside tolerance, max err {err.max()}"
    assert fro <= 1e-2 * rfro + 1e-4 * np.sqrt(ref.size), f"{label}: Frobenius error {fro} of {rfro}"


def run(q, kv, idx, sm, dout, own_forward=False):
    """The backward on the GPU. out/lse: the oracle's forward (out rounded to
    bf16), or with own_forward the library's forward on the same inputs."""
    dsa = _dsa()
    qd, kd, idd, dod = q.to(DEV), kv.to(DEV), idx.to(DEV), dout.to(DEV)
    if own_forward:
        out, lse = dsa.sparse_mla_fwd(qd, kd, idd, sm)
    else:
        o, l = sparse_mla_fwd_ref(np64(q), np64(kv), idx.cpu().numpy(), sm)
        out = torch.from_numpy(o).to(torch.bfloat16).to(DEV)
        lse = torch.from_numpy(l).float().to(DEV)
    dq, dkv = dsa.sparse_mla_bwd(qd, kd, idd, sm, out, lse, dod)
    torch.cuda.synchronize()
    return dq, dkv


def kv_major(H, N, topk, T=64):
    """The schedule the library reports for these sizes (its workspace query):
    the kv-major pass takes at most 16 heads, at most 262144 kv rows, and
    topk at least 3/256 of H x num_kv."""
    return _dsa().bwd_workspace_size(T, H, N, topk)[0] == "kv-major"


def ref(q, kv, idx, sm, dout):
    return sparse_mla_bwd_ref(np64(q), np64(kv), idx.cpu().numpy(), sm, np64(dout))


def random_case(T, H, N, topk, seed, pad_frac=0.3, junk=True, dup=True):
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((N, 576), generator=g).to(torch.bfloat16)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    idx = rng.integers(0, N, size=(T, topk)).astype(np.int32)
    if not dup:
        idx = np.stack([rng.permutation(N)[:topk] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, topk)) < pad_frac] = -1
    if junk:
        j = rng.random((T, topk)) < 0.05
        idx[j] = rng.choice(np.array([N, N + 3, -7], dtype=np.int64), size=int(j.sum())).astype(np.int32)
    return q, kv, torch.from_numpy(idx), dout


@pytest.mark.parametrize("H", [1, 8, 16, 17, 48, 64])
def test_bwd_head_counts(H):
    q, kv, idx, dout = random_case(48, H, 300, 100, seed=H)
    dq, dkv = run(q, kv, idx, 1 / 24, dout)
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(np64(dq), rdq, f"dq H={H}")
    check_grad(np64(dkv), rdkv, f"dkv H={H}")


@pytest.mark.parametrize("topk", [1, 31, 33, 64, 2049, 4500])
def test_bwd_topk_and_segments(topk):
    """Ragged last tiles, a single key, and rows longer than one 2048-entry segment."""
    q, kv, idx, dout = random_case(24, 8, 5000, topk, seed=100 + topk)
    dq, dkv = run(q, kv, idx, 1 / 24, dout)
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(np64(dq), rdq, f"dq topk={topk}")
    check_grad(np64(dkv), rdkv, f"dkv topk={topk}")


def test_bwd_empty_rows_and_untouched_kv():
    q, kv, idx, dout = random_case(16, 8, 400, 64, seed=7, dup=False)
    idx[3] = -1                        # a token with no key
    idx[9, :] = 450                    # only out-of-range values
    dq, dkv = run(q, kv, idx, 1 / 24, dout)
    dq, dkv = np64(dq), np64(dkv)
    assert np.all(dq[3] == 0) and np.all(dq[9] == 0)
    named = set(int(v) for v in idx.numpy().ravel() if 0 <= v < 400)
    untouched = [r for r in range(400) if r not in named]
    assert len(untouched) > 0 and np.all(dkv[untouched] == 0)
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(dq, rdq, "dq empty rows")
    check_grad(dkv, rdkv, "dkv empty rows")


def test_bwd_duplicates_add_up():
    """A row named twice by one token gets twice that token's contribution."""
    q, kv, idx, dout = random_case(8, 8, 200, 40, seed=11, pad_frac=0.0, junk=False, dup=False)
    idx2 = idx.clone()
    idx2[:, 20:] = idx[:, :20]         # the first 20 entries, twice each
    dq, dkv = run(q, kv, idx2, 1 / 24, dout)
    rdq, rdkv = ref(q, kv, idx2, 1 / 24, dout)
    check_grad(np64(dq), rdq, "dq duplicates")
    check_grad(np64(dkv), rdkv, "dkv duplicates")


def test_bwd_swe_workload_full():
    """The SWE-like prefill (2119 tokens, 8 heads, topk 2048, shuffled -1
    padding) at full size, every token and every kv row checked."""
    d = workloads.make_flat("swe")
    g = torch.Generator().manual_seed(5)
    dout = torch.randn((d["q"].shape[0], 8, 512), generator=g).to(torch.bfloat16)
    dq, dkv = run(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    rdq, rdkv = ref(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    check_grad(np64(dq), rdq, "dq swe")
    check_grad(np64(dkv), rdkv, "dkv swe")


def test_bwd_after_own_forward_swe():
    """End to end: the library's forward, then its backward, on the full
    SWE-like prefill."""
    d = workloads.make_flat("swe")
    g = torch.Generator().manual_seed(9)
    dout = torch.randn((d["q"].shape[0], 8, 512), generator=g).to(torch.bfloat16)
    dq, dkv = run(d["q"], d["kv"], d["indices"], d["sm_scale"], dout, own_forward=True)
    rdq, rdkv = ref(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    check_grad(np64(dq), rdq, "dq swe end to end", elem_tol=1e-1)
    check_grad(np64(dkv), rdkv, "dkv swe end to end", elem_tol=1e-1)


def test_bwd_wide_heads_small():
    d = workloads.make_flat("wide", num_tokens=160, topk=2048)
    g = torch.Generator().manual_seed(6)
    dout = torch.randn((160, 64, 512), generator=g).to(torch.bfloat16)
    dq, dkv = run(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    rdq, rdkv = ref(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    check_grad(np64(dq), rdq, "dq wide160")
    check_grad(np64(dkv), rdkv, "dkv wide160")


def test_bwd_strided_and_many_heads():
    """Strided q (every other head of a wider tensor), kv rows 640 apart, an
    index row with trailing columns, dq/dkv views into larger buffers; and
    128 heads (eight head blocks)."""
    T, H, N, k = 20, 128, 500, 150
    q_big, kv, idx, dout = random_case(T, 2 * H, N, k, seed=21)
    dout = dout[:, :H].contiguous()
    q = q_big[:, ::2]
    kv_big = torch.zeros((N, 640), dtype=torch.bfloat16)
    kv_big[:, :576] = kv
    idx_big = torch.full((T, k + 8), -1, dtype=torch.int32)
    idx_big[:, :k] = idx
    dsa = _dsa()
    qd = q_big.to(DEV)[:, ::2]
    kvd = kv_big.to(DEV)[:, :576]
    idd = idx_big.to(DEV)[:, :k]
    o, l = sparse_mla_fwd_ref(np64(q), np64(kv), idx.numpy(), 1 / 24)
    out = torch.from_numpy(o).to(torch.bfloat16).to(DEV)
    lse = torch.from_numpy(l).float().to(DEV)
    dq_big = torch.full((T, H, 640), 7.0, device=DEV)
    dkv_big = torch.full((N, 600), 7.0, device=DEV)
    dq, dkv = dsa.sparse_mla_bwd(qd, kvd, idd, 1 / 24, out, lse, dout.to(DEV),
                                 dq=dq_big[:, :, :576], dkv=dkv_big[:, :576])
    torch.cuda.synchronize()
    assert (dq_big[:, :, 576:] == 7.0).all() and (dkv_big[:, 576:] == 7.0).all()
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(np64(dq), rdq, "dq strided H=128")
    check_grad(np64(dkv), rdkv, "dkv strided H=128")


@pytest.mark.parametrize("H", [1, 5, 8, 16])
def test_bwd_kv_major_pass(H):
    """The kv-major pass: 150 tokens (three 64-token chunks, the last ragged),
    200 kv rows (seven 32-row blocks, the last with 8 rows), distinct entries
    with -1 and out-of-range values; a token with no key, a token with only
    out-of-range values, and two tokens that name a row twice (those two go
    to the token-major kernel inside the same call)."""
    T, N, topk = 150, 200, 160
    assert kv_major(H, N, topk)
    q, kv, idx, dout = random_case(T, H, N, topk, seed=300 + H, dup=False)
    idx[4] = -1
    idx[9] = 213
    idx[40, 0] = idx[40, 1] = 17           # duplicate pair
    idx[141, 5] = idx[141, 100] = 199      # duplicate of the last row
    dq, dkv = run(q, kv, idx, 1 / 24, dout)
    dq, dkv = np64(dq), np64(dkv)
    assert np.all(dq[4] == 0) and np.all(dq[9] == 0)
    named = set(int(v) for v in idx.numpy().ravel() if 0 <= v < N)
    untouched = [r for r in range(N) if r not in named]
    assert np.all(dkv[untouched] == 0)
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(dq, rdq, f"dq kv-major H={H}")
    check_grad(dkv, rdkv, f"dkv kv-major H={H}")


def test_bwd_kv_major_causal_rows():
    """Dense causal rows (token t names 0..t in shuffled order): every pair of
    the lower triangle, blocks named by one token only at the diagonal."""
    d = workloads.make_flat("swe", num_tokens=333, topk=512)
    T, H = d["q"].shape[:2]
    N = d["kv"].shape[0]
    assert kv_major(H, N, 512)
    g = torch.Generator().manual_seed(12)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    dq, dkv = run(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    rdq, rdkv = ref(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    check_grad(np64(dq), rdq, "dq causal kv-major")
    check_grad(np64(dkv), rdkv, "dkv causal kv-major")


def test_bwd_paths_of_the_cases():
    """The cases above reach every schedule: the token-major kernel for sparse
    rows (5000 kv rows, topk up to 64), the kv-major pass for the SWE-like
    rows and the small dense cases at up to 16 heads, the split schedule
    above 16 heads."""
    assert not kv_major(8, 5000, 64) and not kv_major(8, 5000, 1) and kv_major(8, 5000, 2049)
    assert kv_major(8, 300, 100) and kv_major(16, 300, 100) and not kv_major(17, 300, 100)
    d = workloads.make_flat("swe")
    assert kv_major(d["q"].shape[1], d["kv"].shape[0], d["indices"].shape[1])
    assert not kv_major(64, 300, 100)
    # above 16 heads: the split schedule for the small cases, the wide and
    # packed workloads; the token-major kernel for rows sparser than that
    assert split(17, 300, 100) and split(48, 300, 100) and split(64, 300, 100) and split(128, 500, 150)
    assert split(64, 8192, 2048, 8192) and split(64, 16384, 2048, 16384) and split(64, 32768, 2048, 32768)
    assert not split(64, 5000, 64) and not split(16, 300, 100)


@pytest.mark.parametrize("N", [262144, 262145])
def test_bwd_kv_major_size_limit(N):
    """The kv-major schedule's limits: 262144 kv rows (8192 mask words, the
    prepass's whole LDS bitmap) with 3 N H = 256 topk exactly takes it; one
    row more takes the token-major kernel. Both against the oracle."""
    T, H, topk = 3, 1, 3072
    assert kv_major(H, N, topk) == (N == 262144)
    rng = np.random.default_rng(N)
    g = torch.Generator().manual_seed(N)
    q = torch.randn((T, H, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((N, 576), generator=g).to(torch.bfloat16)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    planted = np.array([0, N - 1, N - 2, 31, 32])   # first and last rows, a block edge
    rows = [np.concatenate([planted, rng.choice(np.setdiff1d(np.arange(N), planted), topk - 5, replace=False)])]
    rows += [rng.choice(N, topk, replace=False) for _ in range(T - 1)]
    idx = torch.from_numpy(np.stack(rows).astype(np.int32))
    dq, dkv = run(q, kv, idx, 1 / 24, dout)
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(np64(dq), rdq, f"dq N={N}")
    named = np.unique(idx.numpy())
    named_t = torch.from_numpy(named).long().to(dkv.device)
    check_grad(np64(dkv[named_t]), rdkv[named], f"dkv N={N} (named rows)")
    unnamed = torch.ones(N, dtype=torch.bool, device=dkv.device)
    unnamed[named_t] = False
    assert bool((dkv[unnamed] == 0).all())


def test_bwd_kv_major_strided():
    """The kv-major schedule on strided views: q every other head of a wider
    tensor, kv rows 640 apart, index rows with trailing columns, dO a head
    slice, dq and dkv views into larger buffers that must stay untouched
    outside the views."""
    T, H, N, k = 100, 8, 150, 120
    assert kv_major(H, N, k)
    q_big, kv, idx, dout_big = random_case(T, 2 * H, N, k, seed=31, dup=False)
    q = q_big[:, ::2]
    dout = dout_big[:, 3:3 + H]
    kv_big = torch.zeros((N, 640), dtype=torch.bfloat16)
    kv_big[:, :576] = kv
    idx_big = torch.full((T, k + 8), 7, dtype=torch.int32)
    idx_big[:, :k] = idx
    dsa = _dsa()
    qd = q_big.to(DEV)[:, ::2]
    dod = dout_big.to(DEV)[:, 3:3 + H]
    kvd = kv_big.to(DEV)[:, :576]
    idd = idx_big.to(DEV)[:, :k]
    o, l = sparse_mla_fwd_ref(np64(q), np64(kv), idx.numpy(), 1 / 24)
    out = torch.from_numpy(o).to(torch.bfloat16).to(DEV)
    lse = torch.from_numpy(l).float().to(DEV)
    dq_big = torch.full((T, H, 640), 7.0, device=DEV)
    dkv_big = torch.full((N, 600), 7.0, device=DEV)
    dq, dkv = dsa.sparse_mla_bwd(qd, kvd, idd, 1 / 24, out, lse, dod,
                                 dq=dq_big[:, :, :576], dkv=dkv_big[:, :576])
    torch.cuda.synchronize()
    assert (dq_big[:, :, 576:] == 7.0).all() and (dkv_big[:, 576:] == 7.0).all()
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(np64(dq), rdq, "dq strided kv-major")
    check_grad(np64(dkv), rdkv, "dkv strided kv-major")


def test_bwd_kv_major_long_causal_rows():
    """Causal rows longer than topk (token t names 256 of its t + 1 keys once
    t > 255, tail padding before that): sparser blocks than the dense causal
    case, still on the kv-major schedule at 8 heads."""
    d = workloads.make_flat("wide", num_tokens=600, num_heads=8, topk=256)
    T, H = d["q"].shape[:2]
    N = d["kv"].shape[0]
    assert kv_major(H, N, 256)
    g = torch.Generator().manual_seed(13)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    dq, dkv = run(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    rdq, rdkv = ref(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    check_grad(np64(dq), rdq, "dq long causal kv-major")
    check_grad(np64(dkv), rdkv, "dkv long causal kv-major")


def split(H, N, topk, T=64):
    """The split schedule (more than 16 heads and num_kv <= 16 topk), as the
    library's workspace query reports it."""
    return _dsa().bwd_workspace_size(T, H, N, topk)[0] == "split"


@pytest.mark.parametrize("H", [17, 32, 33, 64, 128])
def test_bwd_split_schedule(H):
    """The split schedule: 300 tokens (five 64-token chunks of the dkv pass,
    the last ragged), 200 kv rows (one 256-row block that runs past them),
    distinct entries with -1 and out-of-range values; a token with no key, a
    token with only out-of-range values, and two tokens that name a row twice
    (those two take the full token-major kernel inside the same call). Head
    counts that fill one or several 32-head groups, and ones that pad them."""
    T, N, topk = 300, 200, 160
    assert split(H, N, topk)
    q, kv, idx, dout = random_case(T, H, N, topk, seed=400 + H, dup=False)
    idx[4] = -1
    idx[9] = 213
    idx[40, 0] = idx[40, 1] = 17           # duplicate pair
    idx[290, 5] = idx[290, 100] = 199      # duplicate of the last row
    dq, dkv = run(q, kv, idx, 1 / 24, dout)
    dq, dkv = np64(dq), np64(dkv)
    assert np.all(dq[4] == 0) and np.all(dq[9] == 0)
    named = set(int(v) for v in idx.numpy().ravel() if 0 <= v < N)
    untouched = [r for r in range(N) if r not in named]
    assert np.all(dkv[untouched] == 0)
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(dq, rdq, f"dq split H={H}")
    check_grad(dkv, rdkv, f"dkv split H={H}")


@pytest.mark.parametrize("H", [32, 64])
def test_bwd_split_long_rows(H):
    """The split schedule on rows of 4500 entries, three 2048-entry index
    segments per token in the dq pass (32 heads per workgroup at H = 32, 64
    at H = 64), with -1 and out-of-range values making the segments ragged."""
    T, N, topk = 40, 5000, 4500
    assert split(H, N, topk, T)
    q, kv, idx, dout = random_case(T, H, N, topk, seed=700 + H, dup=False)
    dq, dkv = run(q, kv, idx, 1 / 24, dout)
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(np64(dq), rdq, f"dq split long rows H={H}")
    check_grad(np64(dkv), rdkv, f"dkv split long rows H={H}")


def test_bwd_split_causal_rows():
    """Causal rows at 64 heads (token t names min(t + 1, 256) of its keys 0..t,
    tail padding): blocks named by every later token, by a quarter of them,
    and at the diagonal by one token."""
    d = workloads.make_flat("wide", num_tokens=520, topk=256)
    T, H = d["q"].shape[:2]
    assert split(H, d["kv"].shape[0], 256)
    g = torch.Generator().manual_seed(14)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    dq, dkv = run(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    rdq, rdkv = ref(d["q"], d["kv"], d["indices"], d["sm_scale"], dout)
    check_grad(np64(dq), rdq, "dq causal split")
    check_grad(np64(dkv), rdkv, "dkv causal split")


def test_bwd_split_strided():
    """The split schedule on strided views: q every other head of a wider
    tensor, kv rows 640 apart, index rows with trailing columns, dO a head
    slice, dq and dkv views into larger buffers that stay untouched outside
    the views; 40 heads (a full and a padded head group)."""
    T, H, N, k = 100, 40, 150, 120
    assert split(H, N, k)
    q_big, kv, idx, dout_big = random_case(T, 2 * H, N, k, seed=32, dup=False)
    q = q_big[:, ::2]
    dout = dout_big[:, 3:3 + H]
    kv_big = torch.zeros((N, 640), dtype=torch.bfloat16)
    kv_big[:, :576] = kv
    idx_big = torch.full((T, k + 8), 7, dtype=torch.int32)
    idx_big[:, :k] = idx
    dsa = _dsa()
    qd = q_big.to(DEV)[:, ::2]
    dod = dout_big.to(DEV)[:, 3:3 + H]
    kvd = kv_big.to(DEV)[:, :576]
    idd = idx_big.to(DEV)[:, :k]
    o, l = sparse_mla_fwd_ref(np64(q), np64(kv), idx.numpy(), 1 / 24)
    out = torch.from_numpy(o).to(torch.bfloat16).to(DEV)
    lse = torch.from_numpy(l).float().to(DEV)
    dq_big = torch.full((T, H, 640), 7.0, device=DEV)
    dkv_big = torch.full((N, 600), 7.0, device=DEV)
    dq, dkv = dsa.sparse_mla_bwd(qd, kvd, idd, 1 / 24, out, lse, dod,
                                 dq=dq_big[:, :, :576], dkv=dkv_big[:, :576])
    torch.cuda.synchronize()
    assert (dq_big[:, :, 576:] == 7.0).all() and (dkv_big[:, 576:] == 7.0).all()
    rdq, rdkv = ref(q, kv, idx, 1 / 24, dout)
    check_grad(np64(dq), rdq, "dq strided split")
    check_grad(np64(dkv), rdkv, "dkv strided split")


def test_bwd_varlen16k_full_sampled():
    """The packed-document prefill at full size (16384 tokens in documents,
    64 heads, topk 2048, the split schedule), sampled as the wide case: dq
    of tokens at document edges and mid-document, and dkv of two rows 60
    before the end of every document (each named only by later tokens of
    its own document, about 50 of them), with every token that names them
    given to the oracle."""
    dsa = _dsa()
    d = workloads.make_flat("varlen16k", device=DEV)
    T, H = d["q"].shape[:2]
    N = d["kv"].shape[0]
    assert split(H, N, 2048, T)
    cu = d["cu_seqlens"].numpy()
    dout = workloads.randn_bf16((T, H, 512), 78, DEV)
    idx = d["indices"].cpu().numpy()
    rows = np.concatenate([np.arange(int(e) - 60, int(e) - 58) for e in cu[1:]])
    toks = np.array([0, int(cu[1]), int(cu[1]) - 1, int(cu[len(cu) // 2]) + 5, T - 1])
    naming = np.flatnonzero(np.isin(idx, rows).any(axis=1))
    U = np.union1d(naming, toks)
    assert len(U) < 400
    q_u, kv_c = np64(d["q"][torch.from_numpy(U).to(DEV)]), np64(d["kv"])
    o_u, l_u = sparse_mla_fwd_ref(q_u, kv_c, idx[U], d["sm_scale"])
    out, lse = dsa.sparse_mla_fwd(d["q"], d["kv"], d["indices"], d["sm_scale"])
    ut = torch.from_numpy(U).to(DEV)
    out[ut] = torch.from_numpy(o_u).to(torch.bfloat16).to(DEV)
    lse[ut] = torch.from_numpy(l_u).float().to(DEV)
    dq, dkv = dsa.sparse_mla_bwd(d["q"], d["kv"], d["indices"], d["sm_scale"], out, lse, dout)
    torch.cuda.synchronize()
    rdq, rdkv = sparse_mla_bwd_ref(q_u, kv_c, idx[U], d["sm_scale"], np64(dout[ut]))
    check_grad(np64(dq[ut]), rdq, "dq varlen16k sampled tokens")
    check_grad(np64(dkv[torch.from_numpy(rows).to(DEV)]), rdkv[rows], "dkv varlen16k sampled rows")


def test_bwd_wide_full_sampled():
    """The wide-head prefill at full size (8192 tokens, 64 heads, topk 2048,
    the split schedule), in the configuration bench.py --op bwd times, on
    outputs the oracle can compute one by one: dq of sampled tokens (a
    token's dq depends on its own row only) and dkv of sampled kv rows (a
    row's dkv is complete once every token that names it is included).
    out and LSE of those tokens are the oracle's; the other tokens' (which
    reach none of the sampled outputs) are the library's forward."""
    dsa = _dsa()
    d = workloads.make_flat("wide", device=DEV)
    T, H = d["q"].shape[:2]
    N = d["kv"].shape[0]
    assert split(H, N, 2048, T)
    dout = workloads.randn_bf16((T, H, 512), 77, DEV)
    idx = d["indices"].cpu().numpy()
    rows = np.array([8000, 8063, 8064, 8100, 8150, 8191])
    toks = np.array([0, 1, 2047, 2048, 4095, 6000, 8191])
    naming = np.flatnonzero(np.isin(idx, rows).any(axis=1))
    U = np.union1d(naming, toks)
    q_u, kv_c = np64(d["q"][torch.from_numpy(U).to(DEV)]), np64(d["kv"])
    o_u, l_u = sparse_mla_fwd_ref(q_u, kv_c, idx[U], d["sm_scale"])
    out, lse = dsa.sparse_mla_fwd(d["q"], d["kv"], d["indices"], d["sm_scale"])
    ut = torch.from_numpy(U).to(DEV)
    out[ut] = torch.from_numpy(o_u).to(torch.bfloat16).to(DEV)
    lse[ut] = torch.from_numpy(l_u).float().to(DEV)
    dq, dkv = dsa.sparse_mla_bwd(d["q"], d["kv"], d["indices"], d["sm_scale"], out, lse, dout)
    torch.cuda.synchronize()
    rdq, rdkv = sparse_mla_bwd_ref(q_u, kv_c, idx[U], d["sm_scale"], np64(dout[ut]))
    check_grad(np64(dq[ut]), rdq, "dq wide sampled tokens")
    check_grad(np64(dkv[torch.from_numpy(rows).to(DEV)]), rdkv[rows], "dkv wide sampled rows")
