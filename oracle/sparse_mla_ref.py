"""Plain CPU oracle of the DSA sparse MLA forward (prefill and paged decode).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the product path never does.
It shares no code, constants or helpers with the HIP library.

What is computed, and where it comes from
------------------------------------------
* "DSA Sparse MLA" forward that returns an output and an LSE:
  "[Feature] Add optional FlashMLA backend for DSA Sparse MLA"
  (InternLM/xtuner PR 2083), sections Motivation and Runtime constraints.
  Those constraints fix one shared KV row per key (kv_group=1) and a value
  width of 512.
* Shapes: bf16 Q and KV, dqk=576, dv=512, topk=2048, and index rows padded
  with -1: "feat: add XTuner TileLang sparse MLA backend" (InternLM/lmdeploy
  PR 4904), sections Performance > Isolated sparse MLA forward and
  Validation.
* Paged decode reads the BF16 paged cache without a gather copy, after a
  logical-to-physical index mapping: the same lmdeploy page, section Summary
  and the per-file overview (shared index mapping utilities).

Readings where the pages are silent (each is listed with its reason in the
design notes):
* V is the leading 512 of the 576 KV columns (the latent part; the trailing 64
  are the rope part).
* LSE is the natural log of sum_j exp(sm_scale * q . k_j), so it includes the
  softmax scale.
* An index entry is a key iff 0 <= i < N. Anything else (-1 padding or an
  out-of-range value) is skipped. Duplicate entries count with multiplicity.
* A row with no key gives O = 0 and LSE = -inf (log of an empty sum).
* Paged decode: query token t belongs to sequence t // q_per_seq, its indices
  are logical positions p in that sequence, and p maps to physical row
  page_table[b, p // page_size] * page_size + p % page_size of the flattened
  cache. p < 0, p >= seq_lens[b], a page slot past the table, or a page entry
  outside [0, num_pages) is skipped.

Precision: the pages do not fix the oracle's precision, so it computes in
float64 by default (float32 on request, for the noise-floor comparison). bf16
inputs are passed in as float32 or float64 arrays, which hold them exactly.
Library primitives used as steps: numpy matmul, max, exp, sum, log.
"""
from __future__ import annotations

import numpy as np

DQK = 576  # query/key width: 512 latent + 64 rope
DV = 512   # value width: the latent part


def _valid_keys(row: np.ndarray, num_kv: int) -> np.ndarray:
    """Entries of one index row that name a KV row: 0 <= i < N, order kept."""
    row = np.asarray(row, dtype=np.int64)
    return row[(row >= 0) & (row < num_kv)]


def sparse_mla_fwd_ref(q, kv, indices, sm_scale, dtype=np.float64):
    """Sparse MLA forward over a flat KV array.

    q:        [T, H, 576] float array (bf16 values held exactly)
    kv:       [N, 576] float array; one latent row per key, shared by every head
    indices:  [T, topk] integer array of KV row ids; invalid entries are skipped
    sm_scale: softmax scale applied to q . k

    Returns (O [T, H, 512], LSE [T, H]) in `dtype`.

    For each token t and head h, with J the valid entries of indices[t]:
      s_j = sm_scale * sum_d q[t,h,d] * kv[J_j, d]          (d over all 576)
      m   = max_j s_j;  w_j = exp(s_j - m);  l = sum_j w_j
      O[t,h,:] = sum_j w_j * kv[J_j, :512] / l
      LSE[t,h] = m + ln l
    """
    q = np.asarray(q)
    kv = np.asarray(kv)
    indices = np.asarray(indices)
    T, H, D = q.shape
    N = kv.shape[0]
    assert D == DQK and kv.shape[1] == DQK, "rows are 576 wide"
    assert indices.shape[0] == T
    scale = dtype(sm_scale)
    out = np.zeros((T, H, DV), dtype=dtype)
    lse = np.full((T, H), -np.inf, dtype=dtype)
    for t in range(T):
        J = _valid_keys(indices[t], N)
        if J.size == 0:
            continue  # empty key set: O stays 0, LSE stays -inf
        K = kv[J].astype(dtype)               # [|J|, 576] gathered rows
        Qt = q[t].astype(dtype)               # [H, 576]
        S = scale * (Qt @ K.T)                # [H, |J|] scaled scores
        m = S.max(axis=1, keepdims=True)      # per-head max, for stability
        W = np.exp(S - m)                     # unnormalised weights
        l = W.sum(axis=1, keepdims=True)      # softmax denominator
        out[t] = (W @ K[:, :DV]) / l          # V = leading 512 columns
        lse[t] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def map_paged_indices(indices, page_table, seq_lens, num_pages, page_size, q_per_seq):
    """Logical sequence positions -> physical rows of the flattened page cache.

    indices:    [T, topk] logical positions; token t is in sequence t // q_per_seq
    page_table: [S, max_pages] physical page ids
    seq_lens:   [S] tokens held in the cache for each sequence

    Returns [T, topk] int64 physical row ids (page * page_size + offset into
    the [num_pages * page_size, 576] view), with -1 where the entry is skipped.
    """
    p = np.asarray(indices, dtype=np.int64)
    page_table = np.asarray(page_table, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    T = p.shape[0]
    max_pages = page_table.shape[1]
    seq = (np.arange(T) // q_per_seq)[:, None]            # sequence of each token
    ok = (p >= 0) & (p < seq_lens[seq])                   # inside the sequence
    slot = np.where(ok, p // page_size, 0)                # logical page number
    ok &= slot < max_pages                                # inside the table
    page = page_table[seq, np.minimum(slot, max_pages - 1)]
    ok &= (page >= 0) & (page < num_pages)                # a real page
    return np.where(ok, page * page_size + p % page_size, -1)


def sparse_mla_fwd_paged_ref(q, kv_pages, page_table, seq_lens, indices, sm_scale,
                             q_per_seq, dtype=np.float64):
    """Sparse MLA forward over a paged cache: map positions, then the flat form.

    kv_pages: [num_pages, page_size, 576]; the flat view is [num_pages*page_size, 576].
    Other arguments as in map_paged_indices and sparse_mla_fwd_ref.
    """
    kv_pages = np.asarray(kv_pages)
    P, page_size, D = kv_pages.shape
    phys = map_paged_indices(indices, page_table, seq_lens, P, page_size, q_per_seq)
    kv_flat = kv_pages.reshape(P * page_size, D)
    return sparse_mla_fwd_ref(q, kv_flat, phys, sm_scale, dtype=dtype)
