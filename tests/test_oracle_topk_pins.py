"""Pins of the top-k index selection oracle (oracle/topk_ref.py), each
independent of the oracle's own code, and planted mistakes that each fail a pin.

What fixes the result (readings stated in the oracle's header): candidates
key_start <= j < key_end clipped to the score row; at most topk candidates
are all selected unscored (the short-prefill scoring skip of "feat: add
XTuner TileLang sparse MLA backend", per-file overview); otherwise the topk
first in the order (larger score, then smaller column; NaN last; -0 == +0),
listed ascending, then -1.

Pins:
* rank definition (brute force, a different formulation): candidate j is
  selected iff fewer than topk candidates beat it, with "beats" written out as
  scalar comparisons;
* torch.topk on rows of distinct values (a library routine);
* the skip identity: short rows give their whole range, even with NaN scores
  or no scores at all;
* all-equal scores give the first topk columns; special values by hand;
* row format: ascending, inside the range, padded with -1.
"""
from __future__ import annotations

import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle.topk_ref as ref
from oracle import topk_indices_ref


def _beats(sa, ja, sb, jb):
    """True if candidate (score sa, column ja) comes before (sb, jb)."""
    na, nb = math.isnan(sa), math.isnan(sb)
    if na and nb:
        return ja < jb
    if na:
        return False
    if nb:
        return True
    if sa != sb:          # -0.0 == 0.0 here
        return sa > sb
    return ja < jb


def brute_rows(scores, ks, ke, topk, num_cols):
    out = []
    for t in range(len(ks)):
        lo, hi = max(int(ks[t]), 0), min(int(ke[t]), num_cols)
        cand = list(range(lo, hi))
        if len(cand) <= topk:
            sel = cand
        else:
            row = [float(scores[t][j]) for j in cand]
            sel = []
            for a, ja in enumerate(cand):
                rank = sum(1 for b, jb in enumerate(cand) if _beats(row[b], jb, row[a], ja))
                if rank < topk:
                    sel.append(ja)
        out.append(sel + [-1] * (topk - len(sel)))
    return np.array(out, dtype=np.int32)


def _check_format(got, ks, ke, topk, num_cols):
    for t in range(got.shape[0]):
        lo, hi = max(int(ks[t]), 0), min(int(ke[t]), num_cols)
        n = max(hi - lo, 0)
        row = got[t]
        m = min(n, topk)
        assert np.all(row[m:] == -1)
        sel = row[:m]
        assert np.all((sel >= lo) & (sel < hi))
        assert np.all(np.diff(sel) > 0)


# ---------------------------------------------------------------- pins (take the function under test)

def pin_brute_force(fn):
    rng = np.random.default_rng(7)
    for trial in range(40):
        T, C = 6, int(rng.integers(1, 30))
        topk = int(rng.integers(1, 12))
        kind = trial % 3
        if kind == 0:
            s = rng.standard_normal((T, C)).astype(np.float32)
        elif kind == 1:
            s = rng.integers(0, 3, (T, C)).astype(np.float32)          # many ties
        else:
            s = rng.standard_normal((T, C)).astype(np.float32)
            u = rng.random((T, C))
            s[u < 0.1] = np.nan
            s[(u >= 0.1) & (u < 0.2)] = np.inf
            s[(u >= 0.2) & (u < 0.3)] = -np.inf
            s[(u >= 0.3) & (u < 0.4)] = 0.0
            s[(u >= 0.4) & (u < 0.5)] = -0.0
        ks = rng.integers(-3, C, T)
        ke = ks + rng.integers(-2, C + 4, T)
        got = fn(s, ks, ke, topk)
        want = brute_rows(s, ks, ke, topk, C)
        assert np.array_equal(got, want), (trial, got, want)
        _check_format(got, ks, ke, topk, C)


def pin_torch_topk(fn):
    g = torch.Generator().manual_seed(3)
    T, C, topk = 40, 700, 64
    s = torch.randn((T, C), generator=g)
    ks = torch.randint(0, 100, (T,), generator=g)
    ke = ks + torch.randint(65, 600, (T,), generator=g)
    got = fn(s.numpy(), ks.numpy(), ke.numpy(), topk)
    for t in range(T):
        a, b = int(ks[t]), int(ke[t])
        want = set((torch.topk(s[t, a:b], topk).indices + a).tolist())
        assert set(got[t].tolist()) == want


def pin_short_skip(fn):
    T, C, topk = 5, 50, 8
    s = np.full((T, C), np.nan, dtype=np.float32)     # never looked at
    ks = np.array([0, 3, 10, 20, 49])
    ke = np.array([8, 5, 10, 28, 60])                 # 8, 2, 0, 8 and (clipped) 1 candidates
    want = np.full((T, topk), -1, dtype=np.int32)
    want[0] = np.arange(8)
    want[1, :2] = [3, 4]
    want[3] = np.arange(20, 28)
    want[4, 0] = 49
    assert np.array_equal(fn(s, ks, ke, topk), want)
    assert np.array_equal(fn(None, ks, ke, topk, num_cols=C), want)
    # with no scores a row that would need them selects nothing
    got = fn(None, np.array([0]), np.array([9]), topk, num_cols=C)
    assert np.all(got == -1)


def pin_equal_and_special(fn):
    C = 12
    s = np.zeros((1, C), dtype=np.float32)
    assert np.array_equal(fn(s, [2], [12], 4)[0], [2, 3, 4, 5])          # all equal: first columns
    s = np.array([[-0.0, 0.0, 1.0]], dtype=np.float32)
    assert np.array_equal(fn(s, [0], [3], 2)[0], [0, 2])                 # -0 == +0: column 0 first
    s = np.array([[0.0, -0.0, 1.0]], dtype=np.float32)
    assert np.array_equal(fn(s, [0], [3], 2)[0], [0, 2])
    s = np.array([[np.nan, -np.inf, 5.0, np.inf, np.nan]], dtype=np.float32)
    assert np.array_equal(fn(s, [0], [5], 2)[0], [2, 3])                 # inf and 5 beat everything
    assert np.array_equal(fn(s, [0], [5], 3)[0], [1, 2, 3])              # -inf beats NaN
    assert np.array_equal(fn(s, [0], [5], 4)[0], [0, 1, 2, 3])           # then NaN by column
    s = np.array([[3.0, 1.0, 2.0, 2.0, 1.0, 0.0]], dtype=np.float32)
    assert np.array_equal(fn(s, [0], [6], 3)[0], [0, 2, 3])
    assert np.array_equal(fn(s, [0], [6], 4)[0], [0, 1, 2, 3])           # tie 1.0: column 1 before 4
    assert np.array_equal(fn(s, [1], [6], 3)[0], [1, 2, 3])


ALL_PINS = [pin_brute_force, pin_torch_topk, pin_short_skip, pin_equal_and_special]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(topk_indices_ref)


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "ties to the larger column": ("np.lexsort((cand, neg, nan))", "np.lexsort((-cand, neg, nan))"),
    "smallest scores kept": ("neg = np.where(nan, 0.0, -s)", "neg = np.where(nan, 0.0, s)"),
    "NaN first": ("np.lexsort((cand, neg, nan))", "np.lexsort((cand, neg, ~nan))"),
    "skip only below topk": ("if cand.size <= topk:", "if cand.size < topk:"),
    "range end inclusive": ("hi = min(int(key_end), int(num_cols))", "hi = min(int(key_end) + 1, int(num_cols))"),
    "start not clipped": ("lo = max(int(key_start), 0)", "lo = int(key_start)"),
    "rows in score order": ("chosen = np.sort(cand[order[:topk]])", "chosen = cand[order[:topk]]"),
    "-0 below +0": ("neg = np.where(nan, 0.0, -s)",
                    "neg = np.where(nan, 0.0, -s - np.where(np.signbit(s) & (s == 0), -1e-300, 0.0))"),
    "one too few": ("chosen = np.sort(cand[order[:topk]])", "chosen = np.sort(cand[order[:topk - 1]])"),
}


def _mutant(old, new):
    src = inspect.getsource(ref)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("topk_mutant")
    exec(compile(src.replace(old, new), "topk_mutant", "exec"), mod.__dict__)
    return mod.topk_indices_ref


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mutant_fails_a_pin(name):
    fn = _mutant(*MUTANTS[name])
    caught = False
    for pin in ALL_PINS:
        try:
            pin(fn)
        except Exception:
            caught = True
            break
    assert caught, f"no pin catches the mutant: {name}"
