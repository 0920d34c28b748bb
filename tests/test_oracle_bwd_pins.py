"""Pins of the backward oracle to facts outside itself (no GPU needed).

Each pin is a function of the backward oracle callable, so that the mutant
test below can run the same pins against copies with a planted mistake.

Pins (what fixes each part of the backward):
  finite differences  central differences of L = sum(dO * O) through the
                      forward oracle (itself pinned in test_oracle_pins.py),
                      on random q and kv coordinates, latent and rope alike,
                      with duplicates, -1 and out-of-range entries in the rows
  dense causal        full causal index rows reduce the method to dense causal
                      single-KV-head attention: torch autograd through
                      scaled_dot_product_attention in float64 (a library
                      routine), with K = kv[:, :576] and V = kv[:, :512]
  untouched rows      kv rows that no index names get exactly zero gradient
  permutation         order and -1 padding of the index rows change nothing
  heads               permuting query heads permutes dq, leaves dkv
  linearity in dO     the gradients are linear in the upstream gradient
"""
from __future__ import annotations

import inspect
import types

import numpy as np
import pytest
import torch

import oracle.bwd_ref as bref
from oracle import DQK, DV, sparse_mla_bwd_ref, sparse_mla_fwd_ref


def _rand(rng, *shape, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return x.to(torch.bfloat16).float().numpy().astype(np.float64)


def _case(seed, T=3, H=2, N=6, topk=7, scale=0.25):
    rng = np.random.default_rng(seed)
    q = _rand(rng, T, H, DQK)
    kv = _rand(rng, N, DQK)
    dout = _rand(rng, T, H, DV)
    idx = np.array([[0, 2, 2, -1, 5, 9, -3],      # duplicate, -1, out of range
                    [1, -1, -1, -1, -1, -1, -1],  # one key
                    [4, 3, 0, 1, 2, 5, 0]], dtype=np.int64)[:T, :topk]
    return q, kv, idx, scale, dout


# ------------------------------------------------------------------ pins

def pin_finite_differences(bwd):
    q, kv, idx, sm, dout = _case(1)
    dq, dkv = bwd(q, kv, idx, sm, dout)

    def loss(qq, kk):
        o, _ = sparse_mla_fwd_ref(qq, kk, idx, sm)
        return float((o * dout).sum())

    rng = np.random.default_rng(2)
    eps = 1e-5
    coords_q = [(t, h, d) for t in range(3) for h in range(2) for d in (0, 7, 511, 512, 575)]
    coords_q += [tuple(int(v) for v in (rng.integers(3), rng.integers(2), rng.integers(DQK))) for _ in range(30)]
    for t, h, d in coords_q:
        qp, qm = q.copy(), q.copy()
        qp[t, h, d] += eps
        qm[t, h, d] -= eps
        fd = (loss(qp, kv) - loss(qm, kv)) / (2 * eps)
        assert abs(fd - dq[t, h, d]) <= 1e-7 + 1e-6 * abs(fd), ("dq", t, h, d, fd, dq[t, h, d])
    coords_kv = [(r, d) for r in (0, 2, 5) for d in (0, 300, 511, 512, 540, 575)]
    coords_kv += [(int(rng.integers(6)), int(rng.integers(DQK))) for _ in range(30)]
    for r, d in coords_kv:
        kp, km = kv.copy(), kv.copy()
        kp[r, d] += eps
        km[r, d] -= eps
        fd = (loss(q, kp) - loss(q, km)) / (2 * eps)
        assert abs(fd - dkv[r, d]) <= 1e-7 + 1e-6 * abs(fd), ("dkv", r, d, fd, dkv[r, d])


def pin_dense_causal(bwd):
    rng = np.random.default_rng(3)
    T, H = 6, 3
    sm = 0.2
    q = _rand(rng, T, H, DQK)
    kv = _rand(rng, T, DQK)
    dout = _rand(rng, T, H, DV)
    idx = np.full((T, T), -1, dtype=np.int64)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t + 1)
    dq, dkv = bwd(q, kv, idx, sm, dout)

    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(kv, requires_grad=True)
    Q = qt.permute(1, 0, 2)[None]                         # [1, H, T, 576]
    K = kt[None, None].expand(1, H, T, DQK)
    V = kt[None, None, :, :DV].expand(1, H, T, DV)
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=sm)
    (O[0].permute(1, 0, 2) * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dkv, kt.grad.numpy(), rtol=1e-9, atol=1e-11)


def pin_untouched_rows_and_padding(bwd):
    q, kv, idx, sm, dout = _case(4)
    dq, dkv = bwd(q, kv, idx, sm, dout)
    assert np.all(dkv[[r for r in range(kv.shape[0]) if r not in set(idx[idx >= 0].tolist())]] == 0)
    rng = np.random.default_rng(5)
    perm = np.stack([rng.permutation(row) for row in idx])
    wide = np.concatenate([perm, np.full((idx.shape[0], 5), -1), np.full((idx.shape[0], 2), 99)], axis=1)
    dq2, dkv2 = bwd(q, kv, wide, sm, dout)
    np.testing.assert_allclose(dq2, dq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkv2, dkv, rtol=1e-11, atol=1e-12)


def pin_heads(bwd):
    q, kv, idx, sm, dout = _case(6, H=3)
    dq, dkv = bwd(q, kv, idx, sm, dout)
    p = np.array([2, 0, 1])
    dqp, dkvp = bwd(q[:, p], kv, idx, sm, dout[:, p])
    np.testing.assert_allclose(dqp, dq[:, p], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkvp, dkv, rtol=1e-11, atol=1e-12)


def pin_linear_in_dout(bwd):
    q, kv, idx, sm, dout = _case(7)
    _, _, _, _, dout2 = _case(8)
    a = bwd(q, kv, idx, sm, dout)
    b = bwd(q, kv, idx, sm, dout2)
    c = bwd(q, kv, idx, sm, 2.0 * dout - 3.0 * dout2)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2.0 * x - 3.0 * y, rtol=1e-10, atol=1e-12)
    z = bwd(q, kv, idx, sm, np.zeros_like(dout))
    assert all(np.all(x == 0) for x in z)


PINS = [pin_finite_differences, pin_dense_causal, pin_untouched_rows_and_padding, pin_heads,
        pin_linear_in_dout]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_oracle_pin(pin):
    pin(sparse_mla_bwd_ref)


# ------------------------------------------------------------------ mutants

MUTANTS = {
    "D term dropped": ("dS = P * (dP - Dh)", "dS = P * dP"),
    "dq scale dropped": ("dq[t] = scale * (dS @ K)", "dq[t] = dS @ K"),
    "key-use scale dropped": ("rows = scale * (dS.T @ Qt)", "rows = dS.T @ Qt"),
    "value use on trailing columns": ("rows[:, :DV] += P.T @ dO", "rows[:, DQK - DV:] += P.T @ dO"),
    "value use left out": ("rows[:, :DV] += P.T @ dO", "rows[:, :DV] += 0.0"),
    "dS sign": ("dS = P * (dP - Dh)", "dS = P * (Dh - dP)"),
    "duplicates overwrite": ("np.add.at(dkv, J, rows)", "dkv[J] = rows"),
    "weights not normalised": ("P = W / W.sum(axis=1, keepdims=True)", "P = W"),
    "D from the wrong axis": ("Dh = (dO * O).sum(axis=1, keepdims=True)",
                              "Dh = (dO * O).sum(axis=0, keepdims=True)[:, :1]"),
    "rope left out of dq": ("dq[t] = scale * (dS @ K)", "dq[t] = scale * np.pad(dS @ V, ((0, 0), (0, DQK - DV)))"),
}


def _mutant(old, new):
    src = inspect.getsource(bref).replace("from .sparse_mla_ref import", "from oracle.sparse_mla_ref import")
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_backward_mutant(name):
    m = _mutant(*MUTANTS[name])
    caught = 0
    for pin in PINS:
        try:
            pin(m.sparse_mla_bwd_ref)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught += 1
    assert caught > 0, f"no pin fails for mutant: {name}"


def test_unmutated_backward_copy_passes_every_pin():
    m = _mutant("DQK, DV", "DQK, DV")
    for pin in PINS:
        pin(m.sparse_mla_bwd_ref)
