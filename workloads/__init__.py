"""Seeded synthetic inputs shaped like the workloads of the DSA sparse MLA pages.

This module only draws inputs. It holds none of the method's arithmetic and is
shared by the tests, the benchmark and the smoke check; both the HIP library's
callers and the CPU oracle receive exactly the tensors it returns.

Workloads (pages: "feat: add XTuner TileLang sparse MLA backend", sections
Performance > Isolated sparse MLA forward and End-to-end serving; "[Feature]
Add optional FlashMLA backend for DSA Sparse MLA", section Validation, 16K/32K
packing):

  short     64 tokens, 8 heads, KV = the 64 tokens, row t = a random
            permutation of causal keys 0..t, then -1 to topk (tail padding)
  swe       2119 tokens, 8 heads, row t = random distinct subset of size
            min(t+1, topk) of keys 0..t, padded with -1, whole row shuffled
  wide      8192 tokens, 64 heads, as swe but tail padding
  varlen16k 16384 packed tokens, 64 heads, documents of length U{256..4096};
            row t = distinct keys from its own document's causal prefix
  varlen32k the same at 32768 tokens
  decode    64 sequences of length U{4096..65536} in a paged cache (page size
            64, pages a random permutation), 6 query tokens per sequence
            (1 + 5 speculative), 8 heads; row (b, j) = topk distinct logical
            positions of the causal context of query j
  decode_fp8  the same inputs with the cache stored as FP8 MLA rows (656
            bytes: e4m3 latent values with a scale per 128, bf16 rope)

Values: Q and KV are N(0,1) in fp32 from torch.Generator(seed), rounded to
bf16. Index structure comes from numpy.random.default_rng(seed). The softmax
scale is 1/sqrt(576) rounded to fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DQK = 576
TOPK = 2048
SM_SCALE = float(np.float32(1.0 / math.sqrt(DQK)))


@dataclass
class Workload:
    name: str
    kind: str            # "flat" or "paged"
    num_tokens: int
    num_heads: int
    topk: int
    seed: int
    desc: str
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "short": Workload("short", "flat", 64, 8, TOPK, 1,
                      "short prefill sq=skv=64, 8 heads"),
    "swe": Workload("swe", "flat", 2119, 8, TOPK, 2,
                    "SWE-like prefill sq=skv=2119, 8 heads"),
    "wide": Workload("wide", "flat", 8192, 64, TOPK, 3,
                     "wide-head prefill sq=skv=8192, 64 heads"),
    "varlen16k": Workload("varlen16k", "flat", 16384, 64, TOPK, 4,
                          "packed varlen prefill 16384 tokens, 64 heads"),
    "varlen32k": Workload("varlen32k", "flat", 32768, 64, TOPK, 6,
                          "packed varlen prefill 32768 tokens, 64 heads"),
    "decode": Workload("decode", "paged", 64 * 6, 8, TOPK, 5,
                       "paged bf16 decode, 64 seqs x 6 query tokens, 8 heads",
                       {"num_seqs": 64, "q_per_seq": 6, "page_size": 64,
                        "min_len": 4096, "max_len": 65536}),
    # the decode workload with its cache stored as FP8 MLA rows (same seeds)
    "decode_fp8": Workload("decode_fp8", "paged_fp8", 64 * 6, 8, TOPK, 5,
                           "paged FP8-cache decode, 64 seqs x 6 query tokens, 8 heads",
                           {"num_seqs": 64, "q_per_seq": 6, "page_size": 64,
                            "min_len": 4096, "max_len": 65536}),
}


def randn_bf16(shape, seed: int, device="cpu", chunk_rows: int = 1 << 14) -> torch.Tensor:
    """N(0,1) fp32 draws from torch.Generator(seed), rounded to bf16.

    Drawn in chunks of the leading dimension so a large array never exists in
    fp32 all at once. The chunking is part of the recipe: the same seed and
    shape give the same bytes on a given device type.
    """
    shape = tuple(int(s) for s in shape)
    gen = torch.Generator(device=device).manual_seed(int(seed))
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + shape[1:], generator=gen,
                                 device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


# ---------------------------------------------------------------- index rows

def causal_rows(rng, num_tokens, topk, layout="tail", starts=None, full_perm=False):
    """Index rows whose keys are drawn from each token's causal prefix.

    Token t at position p in a document that starts at row s gets
    min(p+1, topk) distinct keys from s..s+p (s = 0 without documents).
    layout "tail" puts the -1 padding after the keys; "shuffled" shuffles the
    whole row. full_perm draws a permutation of the whole prefix (it must
    then fit in topk).
    """
    rows = np.full((num_tokens, topk), -1, dtype=np.int32)
    if starts is None:
        starts = np.zeros(num_tokens, dtype=np.int64)
    for t in range(num_tokens):
        s = int(starts[t])
        p = t - s
        n = min(p + 1, topk)
        if full_perm:
            assert p + 1 <= topk
            sel = rng.permutation(p + 1)
        else:
            sel = rng.choice(p + 1, n, replace=False)
        rows[t, :n] = sel + s
        if layout == "shuffled":
            rng.shuffle(rows[t])
    return rows


def document_starts(rng, num_tokens, lo=256, hi=4096):
    """Pack documents of length U{lo..hi} until num_tokens; truncate the last.

    Returns (cu_seqlens, start row of each token's document).
    """
    lens = []
    total = 0
    while total < num_tokens:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, num_tokens - total)
        lens.append(n)
        total += n
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    starts = np.repeat(cu[:-1], lens)
    return cu, starts


# ---------------------------------------------------------------- workloads

def make_flat(name: str, device="cpu", layout=None, num_tokens=None, num_heads=None,
              topk=None, seed=None):
    """Inputs of a flat (prefill) workload; sizes may be overridden for tests.

    Returns a dict with q [T,H,576] bf16, kv [T,576] bf16, indices [T,topk]
    int32 (all on `device`), sm_scale, and cu_seqlens for packed workloads.
    """
    w = WORKLOADS[name]
    T = w.num_tokens if num_tokens is None else int(num_tokens)
    H = w.num_heads if num_heads is None else int(num_heads)
    k = w.topk if topk is None else int(topk)
    s = w.seed if seed is None else int(seed)
    rng = np.random.default_rng(s)
    cu = None
    if name == "short":
        rows = causal_rows(rng, T, k, layout or "tail", full_perm=(T <= k))
    elif name == "swe":
        rows = causal_rows(rng, T, k, layout or "shuffled")
    elif name == "wide":
        rows = causal_rows(rng, T, k, layout or "tail")
    elif name.startswith("varlen"):
        cu, starts = document_starts(rng, T)
        rows = causal_rows(rng, T, k, layout or "tail", starts=starts)
    else:
        raise KeyError(name)
    q = randn_bf16((T, H, DQK), s, device)
    kv = randn_bf16((T, DQK), s + 1000, device)
    out = {"q": q, "kv": kv, "indices": torch.from_numpy(rows).to(device),
           "sm_scale": SM_SCALE}
    if cu is not None:
        out["cu_seqlens"] = torch.from_numpy(cu)
    return out


def _decode_lengths(rng, num_seqs, lo, hi):
    return rng.integers(lo, hi + 1, size=num_seqs).astype(np.int64)


def decode_lengths():
    """Cached lengths L_b of the decode workload's sequences (the first draw
    of its recipe), without building its cache."""
    w = WORKLOADS["decode"]
    e = w.extra
    return _decode_lengths(np.random.default_rng(w.seed), e["num_seqs"], e["min_len"], e["max_len"])


def varlen_cu_seqlens(name: str):
    """Document boundaries of a packed workload (the first draw of its
    recipe), without building its tensors."""
    w = WORKLOADS[name]
    cu, _ = document_starts(np.random.default_rng(w.seed), w.num_tokens)
    return cu


def make_paged(device="cpu", num_seqs=None, q_per_seq=None, num_heads=None, topk=None,
               page_size=None, min_len=None, max_len=None, seed=None, max_pages=None):
    """Inputs of the paged-decode workload; sizes may be overridden for tests.

    Sequence b holds L_b ~ U{min_len..max_len} tokens in ceil(L_b/page_size)
    pages; the physical pages of all sequences are a random permutation of
    0..P-1; unused table slots are -1. Query j of sequence b sits at position
    L_b - q_per_seq + j and its row holds topk distinct logical positions of
    0..L_b - q_per_seq + j (fewer, then -1, if the context is shorter).
    Every slot of every page is N(0,1).
    """
    w = WORKLOADS["decode"]
    e = w.extra
    B = e["num_seqs"] if num_seqs is None else int(num_seqs)
    Q = e["q_per_seq"] if q_per_seq is None else int(q_per_seq)
    H = w.num_heads if num_heads is None else int(num_heads)
    k = w.topk if topk is None else int(topk)
    ps = e["page_size"] if page_size is None else int(page_size)
    lo = e["min_len"] if min_len is None else int(min_len)
    hi = e["max_len"] if max_len is None else int(max_len)
    s = w.seed if seed is None else int(seed)
    rng = np.random.default_rng(s)
    lens = _decode_lengths(rng, B, lo, hi)
    npages = -(-lens // ps)
    P = int(npages.sum())
    mp = int(-(-hi // ps)) if max_pages is None else int(max_pages)
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((B, mp), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += int(npages[b])
    T = B * Q
    rows = np.full((T, k), -1, dtype=np.int32)
    for b in range(B):
        for j in range(Q):
            ctx = int(lens[b]) - Q + j + 1      # positions 0..L_b-Q+j
            n = min(ctx, k)
            if n > 0:
                rows[b * Q + j, :n] = rng.choice(ctx, n, replace=False)
    q = randn_bf16((T, H, DQK), s, device)
    kv_pages = randn_bf16((P, ps, DQK), s + 1000, device, chunk_rows=1 << 10)
    return {"q": q, "kv_pages": kv_pages,
            "page_table": torch.from_numpy(table).to(device),
            "seq_lens": torch.from_numpy(lens.astype(np.int32)).to(device),
            "indices": torch.from_numpy(rows).to(device),
            "q_per_seq": Q, "sm_scale": SM_SCALE}


def make(name: str, device="cpu", **kw):
    """Inputs of any named workload (see the module docstring)."""
    if WORKLOADS[name].kind == "paged":
        return make_paged(device=device, **kw)
    if WORKLOADS[name].kind == "paged_fp8":
        return make_paged_fp8(device=device, **kw)
    return make_flat(name, device=device, **kw)


# ---------------------------------------------------------------- index selection inputs

def causal_ranges(cu_seqlens, num_tokens: int):
    """Candidate ranges of packed causal prefill: token t at position p of the
    document that starts at row d0 may select rows d0 .. d0 + p (itself
    included), as key_start[t] = d0, key_end[t] = d0 + p + 1. Without
    documents (cu_seqlens None) the whole batch is one document."""
    if cu_seqlens is None:
        cu = np.array([0, num_tokens], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    ks = np.zeros(num_tokens, dtype=np.int32)
    ke = np.zeros(num_tokens, dtype=np.int32)
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        ks[a:b] = a
        ke[a:b] = np.arange(a + 1, b + 1)
    return torch.from_numpy(ks), torch.from_numpy(ke)


def index_scores(num_tokens: int, num_cols: int, seed: int, device="cpu", kind="normal"):
    """Stand-in indexer scores, fp32 [num_tokens, num_cols] (the pages do not
    define the score function). kind "normal": N(0,1) from
    torch.Generator(seed); "ties": integers 0..7 drawn the same way (many
    equal scores per row); "special": normal draws with about 1% each of
    +inf, -inf, NaN, +0 and -0 planted by numpy.random.default_rng(seed)."""
    gen = torch.Generator(device=device).manual_seed(int(seed))
    s = torch.randn((num_tokens, num_cols), generator=gen, device=device, dtype=torch.float32)
    if kind == "ties":
        s = torch.floor(s * 2.0 + 4.0).clamp_(0.0, 7.0)
    elif kind == "special":
        rng = np.random.default_rng(seed)
        u = rng.random((num_tokens, num_cols))
        host = s.cpu().numpy()
        for i, v in enumerate((np.inf, -np.inf, np.nan, 0.0, -0.0)):
            host[(u >= 0.01 * i) & (u < 0.01 * (i + 1))] = v
        s = torch.from_numpy(host).to(device)
    elif kind != "normal":
        raise KeyError(kind)
    return s


# ---------------------------------------------------------------- FP8 MLA cache

FP8_ROW_BYTES = 656   # 512 e4m3 latent values, 4 fp32 group scales, 64 bf16 rope values


def quantize_fp8_rows(kv: torch.Tensor) -> torch.Tensor:
    """bf16 rows [..., 576] -> FP8 MLA cache rows uint8 [..., 656], as a cache
    writer would store them: each group of 128 latent values gets the scale
    max|x| / 448 (fp32; 1 for an all-zero group) and its values x / scale
    rounded to e4m3; the 64 rope values are kept in bf16."""
    lead = kv.shape[:-1]
    lat = kv[..., :512].float().reshape(*lead, 4, 128)
    amax = lat.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (lat / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    out = torch.empty((*lead, FP8_ROW_BYTES), dtype=torch.uint8, device=kv.device)
    out[..., :512] = codes.reshape(*lead, 512)
    out[..., 512:528] = scale.reshape(*lead, 4).contiguous().view(torch.uint8)
    out[..., 528:] = kv[..., 512:].contiguous().view(torch.uint8)
    return out


def make_paged_fp8(device="cpu", **kw):
    """The paged-decode inputs (make_paged, same seeds and sizes) with the
    cache stored as FP8 MLA rows: kv_pages becomes uint8 [P, page_size, 656]."""
    d = make_paged(device=device, **kw)
    pages = d["kv_pages"]
    fp8 = torch.empty((*pages.shape[:-1], FP8_ROW_BYTES), dtype=torch.uint8, device=pages.device)
    for p0 in range(0, pages.shape[0], 1024):
        fp8[p0:p0 + 1024] = quantize_fp8_rows(pages[p0:p0 + 1024])
    d["kv_pages"] = fp8
    return d
