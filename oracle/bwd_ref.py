"""Plain CPU oracle of the DSA sparse MLA backward (gradients of the forward).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the product path never does.
It shares no code, constants or helpers with the HIP library.

What is computed, and where it comes from
------------------------------------------
The pages pair the sparse MLA forward with a backward that reuses the
forward's LSE output: "[Feature] Add optional FlashMLA backend for DSA Sparse
MLA" (InternLM/xtuner PR 2083), Motivation (the forward returns an output and
an LSE; the existing backward is kept), and the PrimeIntellect-ai/prime-rl
pull request 4078 that adds a `cudnn_flashmla` DSA backend (its backward is a
separate DSA kernel, timed per call in its measurement table). Neither page
writes the backward out, so this oracle is the plain definition: the exact
gradient of the forward output O with respect to q and kv, for an upstream
gradient dO. The forward itself is the one in sparse_mla_ref.py.

Readings where the pages are silent (each is listed in the design notes):
* The backward takes dO only; LSE is an auxiliary output with no upstream
  gradient of its own.
* kv is one tensor: a key row's gradient gathers both its key use (all 576
  columns) and its value use (the leading 512 columns).
* Masked entries (anything that is not a row id 0 <= i < N) get no gradient;
  duplicate entries count with multiplicity, as in the forward.

With J the valid entries of indices[t], K = kv[J] (|J| x 576), V = K[:, :512],
Q = q[t] (H x 576), and s the forward's scale:
  P   = softmax_j(s * Q K^T)                    (H x |J|)
  O   = P V
  dP  = dO V^T
  D   = rowsum(dO * O)           (= sum_j P_hj dP_hj)
  dS  = P * (dP - D)
  dq[t]         = s * dS K
  dkv[J, :]    += s * dS^T Q      (every row of J, with multiplicity)
  dkv[J, :512] += P^T dO
Library primitives used as steps: numpy matmul, max, exp, sum, add.at.
Precision: float64 by default.
"""
from __future__ import annotations

import numpy as np

from .sparse_mla_ref import DQK, DV, _valid_keys


def sparse_mla_bwd_ref(q, kv, indices, sm_scale, dout, dtype=np.float64):
    """Gradients of the sparse MLA forward.

    q:        [T, H, 576] float array (bf16 values held exactly)
    kv:       [N, 576] float array
    indices:  [T, topk] integer array of KV row ids; invalid entries are skipped
    sm_scale: softmax scale applied to q . k
    dout:     [T, H, 512] upstream gradient of the forward output O

    Returns (dq [T, H, 576], dkv [N, 576]) in `dtype`.
    """
    q = np.asarray(q)
    kv = np.asarray(kv)
    indices = np.asarray(indices)
    dout = np.asarray(dout)
    T, H, D = q.shape
    N = kv.shape[0]
    assert D == DQK and kv.shape[1] == DQK, "rows are 576 wide"
    assert dout.shape == (T, H, DV) and indices.shape[0] == T
    scale = dtype(sm_scale)
    dq = np.zeros((T, H, DQK), dtype=dtype)
    dkv = np.zeros((N, DQK), dtype=dtype)
    for t in range(T):
        J = _valid_keys(indices[t], N)
        if J.size == 0:
            continue  # no key: O is the constant 0, every gradient is 0
        K = kv[J].astype(dtype)               # [|J|, 576]
        V = K[:, :DV]                         # [|J|, 512] values: leading columns
        Qt = q[t].astype(dtype)               # [H, 576]
        dO = dout[t].astype(dtype)            # [H, 512]
        S = scale * (Qt @ K.T)                # [H, |J|]
        W = np.exp(S - S.max(axis=1, keepdims=True))
        P = W / W.sum(axis=1, keepdims=True)  # softmax weights
        O = P @ V                             # [H, 512]
        dP = dO @ V.T                         # [H, |J|]
        Dh = (dO * O).sum(axis=1, keepdims=True)
        dS = P * (dP - Dh)                    # gradient at the scaled scores
        dq[t] = scale * (dS @ K)
        rows = scale * (dS.T @ Qt)            # [|J|, 576] key use
        rows[:, :DV] += P.T @ dO              # value use
        np.add.at(dkv, J, rows)               # duplicates accumulate
    return dq, dkv
