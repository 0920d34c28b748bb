"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host-side validation returns the documented status
before any HIP call is made."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import dsa_sparse_mla_amd as dsa
from dsa_sparse_mla_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_sparse_mla.h")

OK, INVALID, UNSUPPORTED, HIPERR, WORKSPACE = 0, 1, 2, 3, 4
FAKE = 0x10000  # a 64 KiB-aligned non-null address; never dereferenced by the host checks


def fake(i: int) -> int:
    """Distinct fake buffers, 1 TiB apart, so that only the overlap cases overlap."""
    return FAKE + (i << 40)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = dsa.lib()
    names = declared_functions()
    assert "dsa_sparse_mla_fwd" in names and "dsa_sparse_mla_fwd_paged" in names
    for name in names:
        assert hasattr(L, name), f"missing export {name}"


def declared_arg_counts():
    """Parameter count of every function the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    counts = {}
    for name, params in re.findall(r"\b(dsa_\w+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        counts[name] = 0 if params in ("", "void") else params.count(",") + 1
    return counts


def test_binding_prototypes_match_the_header():
    """Each ctypes prototype has as many arguments as the header's declaration."""
    L = dsa.lib()
    counts = declared_arg_counts()
    assert set(counts) == set(declared_functions())
    for name, n in counts.items():
        fn = getattr(L, name)
        assert fn.argtypes is not None, f"{name} has no ctypes prototype"
        assert len(fn.argtypes) == n, f"{name}: binding has {len(fn.argtypes)} arguments, header {n}"


def test_single_hip_runtime_mapped():
    import torch  # noqa: F401
    dsa.lib()
    maps = open("/proc/self/maps").read()
    paths = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(paths) == 1, paths


def test_version_and_status_strings():
    L = dsa.lib()
    assert L.dsa_version() >= 100
    for s in (OK, INVALID, UNSUPPORTED, HIPERR, WORKSPACE, 99):
        assert isinstance(L.dsa_status_string(s), bytes)


def _fwd(**over):
    args = dict(q=fake(0), q_st=8 * 576, q_sh=576, kv=fake(1), kv_st=576, num_kv=100, idx=fake(2),
                idx_st=2048, T=8, H=8, topk=2048, sm=0.04, out=fake(3), o_st=8 * 512, o_sh=512,
                lse=fake(4), lse_st=8, splits=1, ws=None, ws_bytes=0, stream=None)
    args.update(over)
    return dsa.lib().dsa_sparse_mla_fwd(
        args["q"], args["q_st"], args["q_sh"], args["kv"], args["kv_st"], args["num_kv"],
        args["idx"], args["idx_st"], args["T"], args["H"], args["topk"], args["sm"],
        args["out"], args["o_st"], args["o_sh"], args["lse"], args["lse_st"],
        args["splits"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("over,status", [
    ({"T": 0}, OK),                                   # empty batch is a no-op
    ({"T": -1}, INVALID),
    ({"H": 0}, UNSUPPORTED),
    ({"H": 129}, UNSUPPORTED),
    ({"topk": 0}, UNSUPPORTED),
    ({"topk": 65537}, UNSUPPORTED),
    ({"q": None}, INVALID),
    ({"kv": None}, INVALID),
    ({"idx": None}, INVALID),
    ({"out": None}, INVALID),
    ({"lse": None}, INVALID),
    ({"q": fake(0) + 8}, INVALID),                    # q not 16-byte aligned
    ({"kv": fake(1) + 2}, INVALID),
    ({"lse": fake(4) + 2}, INVALID),
    ({"out": fake(0)}, INVALID),                      # out overlaps q
    ({"out": fake(0) + 2 * 8 * 8 * 576 - 16}, INVALID),  # ... by its last 16 bytes
    ({"lse": fake(2) + 4 * 8 * 2048 - 4}, INVALID),   # lse overlaps the last index
    ({"lse": fake(3) + 100}, INVALID),                # lse inside out
    ({"kv": fake(3)}, INVALID),                       # out overlaps kv
    ({"splits": 4, "ws": fake(0), "ws_bytes": 8 * 4 * 8 * 514 * 4}, INVALID),   # workspace over q
    ({"q_sh": 577}, INVALID),                         # stride not a multiple of 8
    ({"kv_st": 572}, INVALID),
    ({"kv_st": 100}, INVALID),                        # rows overlap
    ({"o_sh": 256}, INVALID),
    ({"idx_st": 100}, INVALID),                       # rows shorter than topk
    ({"num_kv": -1}, INVALID),
    ({"sm": float("nan")}, INVALID),
    ({"sm": float("inf")}, INVALID),
    ({"sm": -0.04}, INVALID),                         # the score max is taken before scaling
    ({"splits": -1}, INVALID),
    ({"splits": 3000}, INVALID),                      # more splits than entries
    ({"topk": 5000, "splits": 2}, INVALID),           # fewer than ceil(5000 / 2048)
    ({"splits": 4}, WORKSPACE),                       # a split needs workspace
    ({"splits": 4, "ws": fake(5), "ws_bytes": 100}, WORKSPACE),
    ({"num_kv": 1 << 40}, UNSUPPORTED),               # offsets past 64 GiB
])
def test_fwd_host_validation(over, status):
    assert _fwd(**over) == status


def _paged(**over):
    args = dict(q=fake(0), q_st=8 * 576, q_sh=576, kvp=fake(1), pst=64 * 576, rst=576, P=10, ps=64,
                pt=fake(6), pt_st=16, maxp=16, sl=fake(7), idx=fake(2), idx_st=2048, S=4, Q=2, H=8,
                topk=2048, sm=0.04, out=fake(3), o_st=8 * 512, o_sh=512, lse=fake(4), lse_st=8,
                splits=1, ws=None, ws_bytes=0, stream=None)
    args.update(over)
    a = args
    return dsa.lib().dsa_sparse_mla_fwd_paged(
        a["q"], a["q_st"], a["q_sh"], a["kvp"], a["pst"], a["rst"], a["P"], a["ps"], a["pt"],
        a["pt_st"], a["maxp"], a["sl"], a["idx"], a["idx_st"], a["S"], a["Q"], a["H"], a["topk"],
        a["sm"], a["out"], a["o_st"], a["o_sh"], a["lse"], a["lse_st"], a["splits"], a["ws"],
        a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    ({"S": 0}, OK),
    ({"S": -1}, INVALID),
    ({"Q": 0}, INVALID),
    ({"ps": 48}, UNSUPPORTED),                        # not a power of two
    ({"ps": 8192}, UNSUPPORTED),
    ({"sl": None}, INVALID),
    ({"pt": None}, INVALID),
    ({"pt_st": 8}, INVALID),                          # table rows overlap
    ({"pst": 63 * 576}, INVALID),                     # pages overlap
    ({"kvp": None}, INVALID),
    ({"rst": 576 + 4}, INVALID),
    ({"H": 200}, UNSUPPORTED),
    ({"P": 1 << 40}, UNSUPPORTED),
    ({"lse": fake(6)}, INVALID),                      # lse over the page table
    ({"out": fake(7)}, INVALID),                      # out over seq_lens
    ({"out": fake(1) + 64 * 576 * 2 * 9}, INVALID),   # out inside the last page
])
def test_paged_host_validation(over, status):
    assert _paged(**over) == status


def _bwd(**over):
    args = dict(q=fake(0), q_st=8 * 576, q_sh=576, kv=fake(1), kv_st=576, num_kv=100, idx=fake(2),
                idx_st=2048, T=8, H=8, topk=2048, sm=0.04, out=fake(3), o_st=8 * 512, o_sh=512,
                lse=fake(4), lse_st=8, do=fake(5), do_st=8 * 512, do_sh=512, dq=fake(6), dq_st=8 * 576,
                dq_sh=576, dkv=fake(7), dkv_st=576, ws=None, ws_bytes=0, stream=None)
    args.update(over)
    a = args
    return dsa.lib().dsa_sparse_mla_bwd(
        a["q"], a["q_st"], a["q_sh"], a["kv"], a["kv_st"], a["num_kv"], a["idx"], a["idx_st"],
        a["T"], a["H"], a["topk"], a["sm"], a["out"], a["o_st"], a["o_sh"], a["lse"], a["lse_st"],
        a["do"], a["do_st"], a["do_sh"], a["dq"], a["dq_st"], a["dq_sh"], a["dkv"], a["dkv_st"],
        a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    ({"T": -1}, INVALID),
    ({"H": 0}, UNSUPPORTED),
    ({"H": 129}, UNSUPPORTED),
    ({"topk": 65537}, UNSUPPORTED),
    ({"q": None}, INVALID),
    ({"out": None}, INVALID),
    ({"lse": None}, INVALID),
    ({"do": None}, INVALID),
    ({"dq": None}, INVALID),
    ({"dkv": None}, INVALID),
    ({"kv": None}, INVALID),
    ({"do": fake(5) + 8}, INVALID),                   # dout not 16-byte aligned
    ({"dkv": fake(7) + 4}, INVALID),                  # dkv not 16-byte aligned
    ({"dq": fake(5)}, INVALID),                       # dq over dout
    ({"dkv": fake(6)}, INVALID),                      # dkv over dq
    ({"dkv": fake(1)}, INVALID),                      # dkv over kv
    ({"dq": fake(0) + 16}, INVALID),                  # dq inside q
    ({"dkv_st": 574}, INVALID),                       # not a multiple of 4
    ({"dkv_st": 572}, INVALID),                       # rows overlap
    ({"do_sh": 256}, INVALID),
    ({"dq_sh": 512}, INVALID),                        # dq rows are 576 wide
    ({"do_st": 0}, INVALID),
    ({"sm": float("nan")}, INVALID),
    ({"sm": -1.0}, INVALID),
    ({"num_kv": -1}, INVALID),
    ({"ws_bytes": -1}, INVALID),
    # kv-major sizes (8 heads, 100 rows, topk 2048) need a workspace
    ({"ws": None, "ws_bytes": 0}, WORKSPACE),
    ({"ws": fake(8), "ws_bytes": 100}, WORKSPACE),            # too small
    ({"ws": fake(8) + 16, "ws_bytes": 1 << 20}, WORKSPACE),   # not 256-byte aligned
    ({"ws": fake(6), "ws_bytes": 1 << 20}, INVALID),          # over dq
    ({"ws": fake(1), "ws_bytes": 1 << 20}, INVALID),          # over kv
])
def test_bwd_host_validation(over, status):
    assert _bwd(**over) == status


def test_valid_call_reaches_the_device_check():
    """A well-formed call passes validation; without a GPU the device check fails
    with a HIP status (and nothing is launched). On a GPU machine this test is not
    meaningful, so it only runs where no GPU is visible."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _fwd() in (HIPERR, UNSUPPORTED)
    # out right after q (adjacent, not overlapping) passes the overlap check too
    assert _fwd(out=fake(0) + 2 * 8 * 8 * 576) in (HIPERR, UNSUPPORTED)
    assert _bwd(ws=fake(8), ws_bytes=1 << 20) in (HIPERR, UNSUPPORTED)
    # split sizes (64 heads, 100 kv rows) need a workspace; sparse rows at 64
    # heads (40000 kv rows > 16 x topk) take the token-major kernel and none
    wide = dict(H=64, q_st=64 * 576, o_st=64 * 512, lse_st=64, do_st=64 * 512, dq_st=64 * 576)
    assert _bwd(**wide) == WORKSPACE
    assert _bwd(ws=fake(8), ws_bytes=1 << 20, **wide) == WORKSPACE   # P and s*dS: 4 MiB
    assert _bwd(ws=fake(8), ws_bytes=1 << 23, **wide) in (HIPERR, UNSUPPORTED)
    assert _bwd(num_kv=40000, **wide) in (HIPERR, UNSUPPORTED)


def _bwd_ws(T, H, N, topk):
    return binding.bwd_workspace_size(T, H, N, topk)


def _round256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("T,H,N,topk,schedule", [
    (2119, 8, 2119, 2048, "kv-major"),        # SWE-like prefill rows
    (150, 16, 200, 160, "kv-major"),
    (150, 17, 200, 160, "split"),              # more than 16 heads
    (8192, 64, 8192, 2048, "split"),           # wide-head causal prefill
    (32768, 64, 32768, 2048, "split"),         # num_kv = 16 topk
    (32768, 64, 32769, 2048, "token-major"),   # sparser rows
    (100, 8, 5000, 64, "token-major"),         # sparse rows: 3 N H > 256 topk
    (3, 1, 262144, 3072, "kv-major"),          # 3 N H = 256 topk, the whole LDS bitmap
    (3, 1, 262145, 3072, "token-major"),       # one row more than the bitmap holds
    (0, 8, 100, 2048, "token-major"),          # no tokens
    (10, 8, 0, 2048, "token-major"),           # no kv rows
])
def test_bwd_workspace_query(T, H, N, topk, schedule):
    """The schedule comes from the sizes alone. The kv-major and split
    workspaces start with the occupancy masks and the repeat flags, then the
    kv-major one holds D (16 heads per token); the split one adds the block
    ranks (one per 256 kv rows and token), the entry ranks (topk per token)
    P and s*dS (128 bytes per token, entry and 32-head group) and 256 bytes
    of work-queue counters, each part 256-byte aligned."""
    got, nbytes = _bwd_ws(T, H, N, topk)
    assert got == schedule
    words = (N + 31) // 32
    base = _round256(words * T * 4) + _round256(T * 4) + (T * 16 * 4 if H <= 16 else 0)
    if schedule == "kv-major":
        assert nbytes == base
    elif schedule == "split":
        blk, groups = (words + 7) // 8, (H + 31) // 32
        assert nbytes == (_round256(base) + _round256(blk * T * 4) + _round256(T * topk * 4)
                          + _round256(T * groups * topk * 128) + 256)   # then the dkv queue counters
    else:
        assert nbytes == 0


def test_bwd_workspace_cap():
    """Above 1 GiB of kv-major workspace, or 64 GiB of split workspace, the
    token-major schedule runs instead."""
    T, N = 65536, 131072   # 4096 words x 65536 tokens x 4 bytes = 1 GiB of masks alone
    assert _bwd_ws(T, 1, N, 65536)[0] == "token-major"
    assert _bwd_ws(T // 2, 1, N, 65536)[0] == "kv-major"
    # 64 heads: P and s*dS take 256 bytes per (token, entry); 65536 x 2048 is 32 GiB
    assert _bwd_ws(65536, 64, 32768, 2048)[0] == "split"
    assert _bwd_ws(131072, 64, 32768, 2048)[0] == "token-major"   # 64 GiB and more


def test_bwd_workspace_query_rejects_bad_sizes():
    for args in ((-1, 8, 10, 10), (10, 8, -1, 10), (10, 0, 10, 10), (10, 8, 10, 0)):
        with pytest.raises(binding.DsaError):
            _bwd_ws(*args)


@pytest.mark.parametrize("T,H,topk,req,splits,nbytes", [
    (100, 8, 2048, 1, 1, 0),
    (100, 8, 5000, 0, None, None),
    (10, 64, 2048, 4, 4, 10 * 4 * 64 * 514 * 4),
    (64, 8, 2048, 0, 1, 0),                           # small problems are not split
])
def test_workspace_query(T, H, topk, req, splits, nbytes):
    s, b = binding.workspace_size(T, H, topk, req)
    if splits is not None:
        assert s == splits and b == nbytes
    else:
        assert s >= 3 and b == T * s * H * 514 * 4   # at least ceil(5000 / 2048) splits


@pytest.mark.parametrize("T,H,topk,splits", [
    (384, 8, 2048, 2),      # paged decode: 384 rows fill 2 x 256 CUs only with two splits
    (2119, 8, 2048, 1),     # prefill with enough tokens: never split
    (8192, 64, 2048, 1),
    (130, 8, 2048, 4),      # doubles while tokens x splits < 2 x CUs (130, 260 -> 520)
    (128, 8, 2048, 4),      # 128 x 2048 entries: exactly the size that starts splitting
    (127, 8, 2048, 1),      # one row fewer: too small to pay the merge
    (200, 128, 2048, 2),    # two head blocks count as two workgroups per token
    (100, 8, 4096, 8),      # rows over 2048 entries start at 2 splits, then double
    (3, 8, 60000, 30),      # long rows: ceil(topk / 2048) splits; too few entries to double
    (5, 8, 60000, 60),      # 30 doubles once; 120 would pass the 64-split cap
    (10, 8, 60000, 60),
])
def test_split_policy(T, H, topk, splits):
    """Automatic split count (no GPU here: the host logic assumes 256 CUs,
    the MI355X count): splits double from ceil(topk / 2048) while
    T x head_blocks x splits < 2 x CUs, for calls of at least 256K index
    entries, keeping >= 128 keys per split and at most 64 splits."""
    s, b = binding.workspace_size(T, H, topk, 0)
    assert s == splits
    assert b == (T * s * H * 514 * 4 if s > 1 else 0)


def test_workspace_query_rejects_bad_sizes():
    with pytest.raises(binding.DsaError):
        binding.workspace_size(10, 0, 2048, 0)
    with pytest.raises(binding.DsaError):
        binding.workspace_size(10, 8, 5000, 1)


def _topk(**over):
    args = dict(scores=fake(0), s_st=5000, C=5000, ks=fake(1), ke=fake(2), T=8, topk=2048,
                idx=fake(3), idx_st=2048, stream=None)
    args.update(over)
    a = args
    return dsa.lib().dsa_topk_indices(a["scores"], a["s_st"], a["C"], a["ks"], a["ke"], a["T"], a["topk"],
                                      a["idx"], a["idx_st"], a["stream"])


@pytest.mark.parametrize("over,status", [
    ({"T": -1}, INVALID),
    ({"C": -1}, INVALID),
    ({"s_st": -1}, INVALID),
    ({"idx_st": -1}, INVALID),
    ({"topk": 0}, UNSUPPORTED),
    ({"topk": 65537}, UNSUPPORTED),
    ({"C": 1 << 31}, UNSUPPORTED),          # column ids are int32
    ({"T": 0}, OK),                         # an empty batch is a no-op
    ({"T": 0, "idx": None, "ks": None}, OK),
    ({"ks": None}, INVALID),
    ({"ke": None}, INVALID),
    ({"idx": None}, INVALID),
    ({"idx": fake(3) + 2}, INVALID),        # not 4-byte aligned
    ({"scores": fake(0) + 2}, INVALID),
    ({"idx_st": 2047}, INVALID),            # index rows overlap
    ({"s_st": 4999}, INVALID),              # score rows overlap
    ({"idx": fake(0) + 64}, INVALID),       # indices inside the scores
    ({"idx": fake(1)}, INVALID),            # indices over key_start
])
def test_topk_host_validation(over, status):
    assert _topk(**over) == status


def test_topk_valid_call_reaches_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _topk() in (HIPERR, UNSUPPORTED)
    assert _topk(scores=None, s_st=0) in (HIPERR, UNSUPPORTED)   # no scores is allowed
