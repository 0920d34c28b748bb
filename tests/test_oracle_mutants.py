"""The pins are strong enough: each planted mistake in the oracle fails one.

Every mutant is a copy of the oracle's source with one plausible mistake
(a dropped term, a wrong sign, index or axis, a transposed choice of columns),
executed into a private namespace on the CPU. The real oracle is untouched.
"""
from __future__ import annotations

import inspect
import types

import pytest

import oracle.sparse_mla_ref as ref
import test_oracle_pins as pins

MUTANTS = {
    "V is the trailing 512 columns": ("(W @ K[:, :DV])", "(W @ K[:, DQK - DV:])"),
    "scale dropped": ("S = scale * (Qt @ K.T)", "S = (Qt @ K.T)"),
    "LSE in base 2": ("np.log(l[:, 0])", "np.log2(l[:, 0])"),
    "LSE without the max": ("lse[t] = m[:, 0] + np.log", "lse[t] = np.log"),
    "-1 read as a row id": ("row[(row >= 0) & (row < num_kv)]", "row[(row >= -1) & (row < num_kv)]"),
    "last row dropped": ("row[(row >= 0) & (row < num_kv)]", "row[(row >= 0) & (row < num_kv - 1)]"),
    "duplicates merged": ("return row[(row >= 0) & (row < num_kv)]",
                          "return np.unique(row[(row >= 0) & (row < num_kv)])"),
    "max over the wrong axis": ("m = S.max(axis=1, keepdims=True)", "m = S.max(axis=0, keepdims=True)"),
    "exponent sign": ("W = np.exp(S - m)", "W = np.exp(m - S)"),
    "no normalisation": ("out[t] = (W @ K[:, :DV]) / l", "out[t] = (W @ K[:, :DV])"),
    "rope part left out of the scores": ("S = scale * (Qt @ K.T)", "S = scale * (Qt[:, :DV] @ K[:, :DV].T)"),
    "page offset": ("page * page_size + p % page_size", "page * page_size + p // page_size"),
    "sequence of a token": ("seq = (np.arange(T) // q_per_seq)", "seq = (np.arange(T) % q_per_seq)"),
    "sequence length off by one": ("(p < seq_lens[seq])", "(p <= seq_lens[seq])"),
    "page bound": ("(page < num_pages)", "(page <= num_pages)"),
}


def _mutant(old, new):
    src = inspect.getsource(ref)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _all_pins(m):
    fwd, paged, mapper = m.sparse_mla_fwd_ref, m.sparse_mla_fwd_paged_ref, m.map_paged_indices
    return [
        lambda: pins.pin_hand_worked(fwd),
        lambda: pins.pin_dense_causal(fwd),
        lambda: pins.pin_single_key(fwd),
        lambda: pins.pin_zero_query(fwd),
        lambda: pins.pin_brute_force(fwd),
        lambda: pins.pin_permutation_and_padding(fwd),
        lambda: pins.pin_heads(fwd),
        lambda: pins.pin_peaky(fwd),
        lambda: pins.pin_paged_equals_flat(fwd, paged),
        lambda: pins.pin_page_mapping_by_hand(mapper),
    ]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name):
    old, new = MUTANTS[name]
    m = _mutant(old, new)
    caught = 0
    for pin in _all_pins(m):
        try:
            pin()
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught += 1
    assert caught > 0, f"no pin fails for mutant: {name}"


def test_unmutated_copy_passes_every_pin():
    m = _mutant("DQK = 576", "DQK = 576")
    for pin in _all_pins(m):
        pin()
