"""Scalar-loop implementation of the GQE layer for tiny inputs.

An independent second implementation used only to pin the vectorised
oracle: plain Python floats and loops, no NumPy arithmetic, and different
algorithms for each step (TopK by repeated scans, softmax as a two-pass sum
over visible keys only, slot assembly by explicit index arithmetic).
"""
from __future__ import annotations

import math


def dot(a, b):
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def topk_scan(scores, k):
    """Repeatedly take the first maximum among the remaining entries."""
    chosen = []
    for _ in range(k):
        best = None
        for m, s in enumerate(scores):
            if m in chosen:
                continue
            if best is None or s > scores[best]:
                best = m
        chosen.append(best)
    return sorted(chosen)


def route(x, w_r, G, M, k, b_r=None):
    """x: list of T token vectors; w_r: list of G*M rows. Returns (z, idx, w)."""
    T = len(x)
    z = [[[0.0] * M for _ in range(G)] for _ in range(T)]
    idx = [[None] * G for _ in range(T)]
    w = [[None] * G for _ in range(T)]
    for i in range(T):
        for g in range(G):
            for m in range(M):
                z[i][g][m] = dot(x[i], w_r[g * M + m]) + (b_r[g * M + m] if b_r is not None else 0.0)
            sel = topk_scan(z[i][g], k)
            ex = [math.exp(z[i][g][m]) for m in range(M)]
            tot = sum(ex)
            p = [e / tot for e in ex]
            den = sum(p[m] for m in sel)
            idx[i][g] = sel
            w[i][g] = [p[m] / den for m in sel]
    return z, idx, w


def attend(q, keys, vals, visible):
    """softmax over the visible keys only, written as two passes."""
    d = len(q)
    sc = [dot(q, keys[j]) / math.sqrt(d) for j in range(visible)]
    top = max(sc)
    e = [math.exp(s - top) for s in sc]
    den = sum(e)
    out = [0.0] * len(vals[0])
    for j in range(visible):
        for c in range(len(out)):
            out[c] += e[j] / den * vals[j][c]
    return out


def layer(x, w_r, Q, K, V, W_O, G, k, b_r=None):
    """Q: [S][N+1][d]; K, V: [G][S][d]; x: [S][D]; W_O: [(G*k+2)*d][Dout].

    One sequence. Returns dict with idx, w, A (slot vectors) and y.
    """
    S = len(Q)
    N = len(Q[0]) - 1
    d = len(Q[0][0])
    M = N // G
    z, idx, w = route(x, w_r, G, M, k, b_r)
    A = []
    for i in range(S):
        width = (G * k + 2) * d
        a = [0.0] * width
        obar = [0.0] * d
        for g in range(G):
            for j, m in enumerate(idx[i][g]):
                head = g * M + m
                o = attend(Q[i][head], K[g], V[g], i + 1)
                base = (g * k + j) * d
                for c in range(d):
                    a[base + c] = o[c]
                    obar[c] += w[i][g][j] * o[c]
        s = attend(Q[i][N], K[0], V[0], i + 1)
        for c in range(d):
            a[G * k * d + c] = obar[c]
            a[G * k * d + d + c] = s[c]
        A.append(a)
    Dout = len(W_O[0])
    y = [[sum(A[i][r] * W_O[r][c] for r in range(len(A[i]))) for c in range(Dout)] for i in range(S)]
    return dict(z=z, idx=idx, w=w, A=A, y=y)
