"""Closed forms of causal attention and its gradients when every key of the
KV head is the same vector, for checking whole outputs at sizes the oracle
cannot reach.

With k_j = k for every j, row i's visible scores q_i.k/sqrt(d) are all equal,
so its softmax is uniform: P_ij = 1/(i+1) for j <= i. Then

    lse_i = q_i.k/sqrt(d) + ln(i+1)
    o_i   = mean_{j<=i} v_j
    dV_j  = sum_{i>=j} dO_i/(i+1)
    dK_j  = (1/sqrt(d)) sum_{i>=j} q_i (dO_i.v_j - dO_i.o_i)/(i+1)
    dq_i  = (1/sqrt(d)) k sum_{j<=i} dS_ij = 0

(dS_ij = P_ij (dO_i.v_j - dO_i.o_i) sums to zero over j). The suffix sums
over i >= j run backward over the sequence; the dO_i.v_j term of dK is
split into the part inside a chunk of keys (a masked product) and the part
from later chunks (a d x d running sum), so the cost is linear in S.
"""
from __future__ import annotations

import numpy as np


def _suffix_sum(a: np.ndarray) -> np.ndarray:
    return np.cumsum(a[::-1], axis=0)[::-1]


def stream(q, dO, V, key, chunk: int = 256):
    """One run of rows i = 0..S-1 over a KV head whose keys all equal `key`:
    q, dO: [S, d] (row i's query and output gradient); V: [S, d].
    Returns (lse [S], o [S, d], dK [S, d], dV [S, d]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    key = np.asarray(key, dtype=np.float64)
    S, d = V.shape
    w = 1.0 / np.arange(1, S + 1, dtype=np.float64)
    lse = q @ key / np.sqrt(d) + np.log(np.arange(1, S + 1, dtype=np.float64))
    o = np.cumsum(V, axis=0) * w[:, None]
    delta = np.sum(dO * o, axis=1)
    wdo = dO * w[:, None]
    wq = q * w[:, None]
    dV = _suffix_sum(wdo)
    F = np.zeros((S, d))
    tail = np.zeros((d, d))  # sum over later rows of (w_i q_i) dO_i^T
    for c1 in range(S, 0, -chunk):
        c0 = max(0, c1 - chunk)
        X = np.tril(dO[c0:c1] @ V[c0:c1].T)  # [i, j] = dO_i.v_j where i >= j
        F[c0:c1] = X.T @ wq[c0:c1] + V[c0:c1] @ tail.T
        tail += wq[c0:c1].T @ dO[c0:c1]
    dK = (F - _suffix_sum(wq * delta[:, None])) / np.sqrt(d)
    return lse, o, dK, dV
