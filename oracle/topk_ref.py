"""Plain CPU oracle of the DSA index selection step: score rows -> top-k index rows.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the product path never does.
It shares no code, constants or helpers with the HIP library.

What is computed, and where it comes from
------------------------------------------
* The sparse attention consumes, per query token, a row of topk key ids padded
  with -1 ("feat: add XTuner TileLang sparse MLA backend", InternLM/lmdeploy
  PR 4904, Validation). That page's Summary keeps "DSA index production" for
  short prefill, and its per-file overview describes the indexer's prefill
  scores (computed over chunks of query rows under a logits budget) and a
  short-prefill scoring skip. "[Feature] Add optional FlashMLA backend for DSA
  Sparse MLA" (InternLM/xtuner PR 2083), Changes, reuses an existing indexer
  in front of the sparse kernel.
* Neither page defines the indexer's score function, so scores are an input
  here. This oracle is the step after them: for each query token, keep the
  topk best-scoring candidate keys.

Readings where the pages are silent:
* Token t's candidates are the columns j with key_start[t] <= j < key_end[t]
  of its score row (its causal prefix: in packed prefill the columns from its
  document's first row up to itself; in decode the logical positions of its
  context). Bounds are clipped to [0, num_cols); an empty range selects
  nothing.
* Short-prefill skip: when a token has at most topk candidates, every
  candidate is selected and its scores are not looked at (the page's skip: no
  scoring is needed when the causal prefix is no longer than topk).
* Otherwise the selected set holds the topk candidates that come first in the
  order: larger score first; equal scores (-0 equals +0) by smaller column
  first; NaN after every number (NaNs among themselves by column).
* The row lists the selected column ids in ascending order, then -1 up to
  topk. (The sparse forward does not depend on the order of a row; a fixed
  order makes the result exact to compare.)
* If scores is None, no row is scored: rows with more than topk candidates
  select nothing (all -1).

Library primitives used as steps: numpy lexsort and sort.
"""
from __future__ import annotations

import numpy as np


def _candidates(key_start: int, key_end: int, num_cols: int) -> np.ndarray:
    """Columns key_start .. key_end-1, clipped to the score row."""
    lo = max(int(key_start), 0)
    hi = min(int(key_end), int(num_cols))
    return np.arange(lo, hi, dtype=np.int64) if hi > lo else np.zeros(0, dtype=np.int64)


def topk_indices_ref(scores, key_start, key_end, topk: int, num_cols: int | None = None):
    """Top-k index rows from score rows.

    scores:    [T, num_cols] float32 array, or None (no row is scored)
    key_start: [T] ints, key_end: [T] ints (candidates key_start <= j < key_end)
    topk:      row width of the result (>= 1)
    num_cols:  width of a score row (defaults to scores.shape[1])
    returns int32 [T, topk]: selected column ids ascending, then -1
    """
    key_start = np.asarray(key_start, dtype=np.int64)
    key_end = np.asarray(key_end, dtype=np.int64)
    T = key_start.shape[0]
    if num_cols is None:
        num_cols = scores.shape[1]
    out = np.full((T, topk), -1, dtype=np.int32)
    for t in range(T):
        cand = _candidates(key_start[t], key_end[t], num_cols)
        if cand.size <= topk:                       # short prefix: all of it, unscored
            chosen = cand
        elif scores is None:                        # would need scores that were not given
            continue
        else:
            s = np.asarray(scores[t], dtype=np.float32)[cand].astype(np.float64)
            nan = np.isnan(s)
            neg = np.where(nan, 0.0, -s)            # larger score first; -0 and +0 compare equal
            # lexsort: the last key is primary -> NaN last, then score descending, then column
            order = np.lexsort((cand, neg, nan))
            chosen = np.sort(cand[order[:topk]])
        out[t, :chosen.size] = chosen
    return out

