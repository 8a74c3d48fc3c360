"""Pins that fix the CPU oracle without comparing it to itself.

Each ``pin_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with a value printed on the pages, a closed form, a
reduction to a textbook/library routine, or the scalar brute force. The
mutation test runs every pin against deliberately broken copies of the
oracle to show each plausible mistake is caught by at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _one_token_layer(O, Q, K, V, G, k, z):
    """Run the oracle's routing+attention+assembly for a single token.

    Q: [H+1, d] (last row shared), K, V: [G, d]; z: router scores [G, M].
    """
    H1, d = Q.shape
    M = (H1 - 1) // G
    _, idx, w = O.route_select(np.asarray(z, dtype=np.float64)[None], k)
    Q4 = np.asarray(Q, dtype=np.float64)[None, None]
    K4 = np.asarray(K, dtype=np.float64)[None, :, None, :]
    V4 = np.asarray(V, dtype=np.float64)[None, :, None, :]
    O_r, O_s = O.prefill(Q4, K4, V4, idx.reshape(1, 1, G, k), M)
    A = O.assemble(O_r.reshape(1, G, k, d), w, O_s.reshape(1, d))
    return O_r.reshape(-1), A.reshape(-1)


# --------------------------------------------------------------------------
# Worked examples printed on the pages
# --------------------------------------------------------------------------

def pin_gqa_worked_example(O):
    """GQA example, 4 heads / 2 groups: k = M reduces GQE's hard slot to the
    dense GQA concatenation [1,0,1,0,0,1,0,1]."""
    g = _golden("gqa_worked_example.json")
    Q = np.vstack([np.array(g["Q"], float), [[0.3, -0.7]]])  # + shared head
    hard, _ = _one_token_layer(O, Q, np.array(g["K"], float), np.array(g["V"], float),
                               G=g["G"], k=g["h"] // g["G"], z=np.zeros((g["G"], g["h"] // g["G"])))
    _close(hard, g["concat"], what="GQA worked example")


def pin_mqa_worked_example(O):
    """MQA example: 2 heads sharing one KV head -> [1,0,1,0]."""
    g = _golden("mqa_worked_example.json")
    Q = np.vstack([np.array(g["Q"], float), [[1.0, 0.0]]])
    hard, _ = _one_token_layer(O, Q, np.array(g["K"], float), np.array(g["V"], float),
                               G=1, k=2, z=np.zeros((1, 2)))
    _close(hard, g["concat"], what="MQA worked example")
    assert abs(1.0 / math.sqrt(g["d"]) - g["scaled_score"]) < 1e-4


def pin_three_slot_assembly(O):
    """Derived from the GQA example and the three-part output: with a zero
    router (p = 1/2, 1/2), k=2 gives A = [1,0,1,0,0,1,0,1 | 1,1 | 1,0] and
    k=1 (tie -> expert 0, w = 1) gives A = [1,0,0,1 | 1,1 | 1,0]. The shared
    head reads KV head 0 whatever its query."""
    g = _golden("gqa_worked_example.json")
    Q = np.vstack([np.array(g["Q"], float), [[0.3, -0.7]]])
    K, V = np.array(g["K"], float), np.array(g["V"], float)
    _, A2 = _one_token_layer(O, Q, K, V, G=2, k=2, z=np.zeros((2, 2)))
    _close(A2, [1, 0, 1, 0, 0, 1, 0, 1, 1, 1, 1, 0], what="k=2 slot vector")
    _, A1 = _one_token_layer(O, Q, K, V, G=2, k=1, z=np.zeros((2, 2)))
    _close(A1, [1, 0, 0, 1, 1, 1, 1, 0], what="k=1 slot vector")


def pin_kv_bytes(O):
    for c in _golden("kv_bytes.json")["cases"]:
        got = O.kv_bytes(c["B"], c["L"], c["G"], c["d"], c["S"], c["b"])
        assert got == c["bytes"], f"kv_bytes {c['label']}: {got} != {c['bytes']}"


def pin_nonsquare_causal(O):
    """Queries at positions 5 and 6 over keys 0..6 see 6 and 7 keys. With
    K = 0 (uniform weights) and V_j = j + 10*g, the outputs are the means
    2.5 and 3.0 (+10g); the top-left-triangle bug would give 0 and 0.5."""
    c = _golden("nonsquare_causal.json")
    H, G, L, n = c["H"], c["G"], 2, c["kv_len"]
    M, d = H // G, 4
    K = np.zeros((1, G, n, d))
    V = np.zeros((1, G, n, d))
    for gg in range(G):
        V[0, gg, :, :] = (np.arange(n) + 10.0 * gg)[:, None]
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, L, H + 1, d))
    idx = np.tile(np.arange(M), (1, L, G, 1))  # k = M: every head
    O_r, O_s = O.decode(q, K, V, np.array([n]), idx, M)
    vis = np.array(c["visible_keys"], float)
    want = (vis - 1) / 2.0  # mean of 0..vis-1
    for gg in range(G):
        for j in range(M):
            _close(O_r[0, :, gg, j, 0], want + 10.0 * gg, 1e-12, f"non-square causal g={gg}")
    _close(O_s[0, :, 0], want, 1e-12, "non-square causal shared head")
    # head -> KV mapping of the page
    for h, kv in enumerate(c["head_to_kv"]):
        assert h // M == kv


def pin_decode_left_padding(O):
    """Keys before kv_start are padding: with K = 0 (uniform weights) and
    V_j = j, a query at position p sees the mean of kv_start..p, i.e.
    (kv_start + p) / 2; without the padding mask it would be p / 2."""
    G, H, L, n, d = 2, 4, 2, 9, 3
    M = H // G
    K = np.zeros((2, G, n, d))
    V = np.broadcast_to(np.arange(n, dtype=float)[None, None, :, None], (2, G, n, d)).copy()
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, L, H + 1, d))
    idx = np.tile(np.arange(M), (2, L, G, 1))
    kv_len, kv_start = np.array([9, 6]), np.array([3, 0])
    O_r, O_s = O.decode(q, K, V, kv_len, idx, M, kv_start=kv_start)
    for b in range(2):
        pos = kv_len[b] - L + np.arange(L)
        want = (kv_start[b] + pos) / 2.0
        for g in range(G):
            for j in range(M):
                _close(O_r[b, :, g, j, 0], want, 1e-12, f"left padding b={b}")
        _close(O_s[b, :, 0], want, 1e-12, f"left padding shared b={b}")


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def pin_router_closed_forms(O):
    """z = x W_r^T (+b): one-hot tokens read out router columns; TopK ties go
    to the lower index; w renormalises p over the selected set."""
    rng = np.random.default_rng(5)
    G, M, D = 3, 4, 6
    w_r = rng.standard_normal((G * M, D))
    b_r = rng.standard_normal(G * M)
    x = np.eye(D)
    z = O.route_logits(x, w_r, G, M, b_r)
    for j in range(D):
        _close(z[j].reshape(-1), w_r[:, j] + b_r, 1e-15, "router column read-out")
    # p = [.1,.2,.3,.4] -> top-2 = {2,3}, w = [3/7, 4/7]
    zz = np.log(np.array([[[1.0, 2.0, 3.0, 4.0]]]))
    p, idx, w = O.route_select(zz, 2)
    _close(p[0, 0], [0.1, 0.2, 0.3, 0.4], 1e-15, "softmax of log-probabilities")
    assert idx[0, 0].tolist() == [2, 3]
    _close(w[0, 0], [3 / 7, 4 / 7], 1e-15, "renormalised weights")
    # ties: [1,1,0,1] top-2 -> {0,1}; [0,0,0,0] top-1 -> {0}; top-3 of [2,5,5,5] -> {1,2,3}
    assert O.route_select(np.array([[[1.0, 1.0, 0.0, 1.0]]]), 2)[1][0, 0].tolist() == [0, 1]
    assert O.route_select(np.zeros((1, 1, 4)), 1)[1][0, 0].tolist() == [0]
    assert O.route_select(np.array([[[2.0, 5.0, 5.0, 5.0]]]), 3)[1][0, 0].tolist() == [1, 2, 3]
    # the largest, not the smallest; ascending storage
    assert O.route_select(np.array([[[9.0, -1.0, 4.0, 7.0]]]), 2)[1][0, 0].tolist() == [0, 3]
    # k = 1: w is exactly 1
    _, _, w1 = O.route_select(rng.standard_normal((50, 2, 4)), 1)
    assert np.all(w1 == 1.0)


def pin_single_key_attention(O):
    """With one visible key the softmax weight is 1 and o = v_0 exactly, for
    any query; with two keys and scores a, b the weights are the logistic
    function of (a-b)/sqrt(d)."""
    rng = np.random.default_rng(8)
    d = 4
    K = rng.standard_normal((3, d))
    V = rng.standard_normal((3, d))
    q = rng.standard_normal((1, d))
    _close(O.attend_rows(q, np.array([0]), K, V), V[:1], 1e-15, "one key")
    s = (q @ K[:2].T).ravel() / math.sqrt(d)
    a = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    _close(O.attend_rows(q, np.array([1]), K, V)[0], a * V[0] + (1 - a) * V[1], 1e-14, "two keys")


# --------------------------------------------------------------------------
# Reductions to library routines
# --------------------------------------------------------------------------

def _sdpa(q, k, v):
    """torch CPU scaled_dot_product_attention, causal, fp64. q,k,v: [H,S,d]."""
    with torch.no_grad():
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            is_causal=True)
    return o[0].numpy()


def _rand_qkv(rng, B, S, N, G, d):
    Q = rng.standard_normal((B, S, N + 1, d))
    K = rng.standard_normal((B, G, S, d))
    V = rng.standard_normal((B, G, S, d)) + 10.0 * np.arange(G)[None, :, None, None]
    return Q, K, V


def pin_repeat_kv_equivalence(O):
    """k = M (every expert selected) turns the hard slots into dense GQA.
    Explicit head mapping must equal attention on np.repeat-expanded K/V
    (the page's mapping-vs-repeat check, here with the causal mask), and
    torch's causal SDPA on the repeated K/V."""
    rng = np.random.default_rng(11)
    for (B, S, N, G, d) in [(2, 9, 8, 2, 4), (1, 13, 6, 3, 8)]:
        M = N // G
        Q, K, V = _rand_qkv(rng, B, S, N, G, d)
        idx = np.broadcast_to(np.arange(M), (B, S, G, M)).copy()
        O_r, O_s = O.prefill(Q, K, V, idx, M)
        for b in range(B):
            Kr = np.repeat(K[b], M, axis=0)  # [N, S, d]
            Vr = np.repeat(V[b], M, axis=0)
            q = Q[b, :, :N, :].transpose(1, 0, 2)  # [N, S, d]
            sc = q @ Kr.transpose(0, 2, 1) / np.sqrt(d)
            sc = np.where(np.tril(np.ones((S, S), bool))[None], sc, -np.inf)
            sc = np.exp(sc - sc.max(-1, keepdims=True))
            ref = (sc / sc.sum(-1, keepdims=True)) @ Vr  # [N, S, d]
            got = O_r[b].reshape(S, N, d).transpose(1, 0, 2)
            _close(got, ref, 1e-12, "mapping vs repeat-KV")
            _close(got, _sdpa(q, Kr, Vr), 1e-12, "mapping vs torch SDPA")
            _close(O_s[b], _sdpa(Q[b, :, N][None], K[b, :1], V[b, :1])[0], 1e-12, "shared head vs SDPA")


def pin_mha_mqa_reductions(O):
    """G = H (M = 1, k = 1) is MHA: slot g is head g on its own KV head and
    ō is the plain sum of all heads. G = 1 is MQA: every head reads KV 0."""
    rng = np.random.default_rng(12)
    B, S, d = 1, 7, 4
    for N, G in [(4, 4), (4, 1)]:
        M = N // G
        k = M
        Q, K, V = _rand_qkv(rng, B, S, N, G, d)
        D = 5
        x = rng.standard_normal((B * S, D))
        w_r = rng.standard_normal((N, D))
        W_O = rng.standard_normal(((G * k + 2) * d, 3))
        out = O.layer(x, w_r, Q, K, V, W_O, G, k)
        kvmap = np.arange(N) // M
        heads = np.stack([_sdpa(Q[0, :, h][None], K[0, kvmap[h]][None], V[0, kvmap[h]][None])[0]
                          for h in range(N)], axis=1)  # [S, N, d]
        _close(out["O_r"][0].reshape(S, N, d), heads, 1e-12, f"N={N} G={G} head outputs")
        if M == 1:
            A = O.assemble(out["O_r"].reshape(S, G, 1, d), out["w"], out["O_s"].reshape(S, d))
            _close(A[:, G * d:G * d + d], heads.sum(1), 1e-12, "MHA: ō is the sum of heads")


# --------------------------------------------------------------------------
# Brute force and invariants
# --------------------------------------------------------------------------

def pin_bruteforce(O):
    """Scalar loops on tiny inputs match the vectorised oracle to 1e-12."""
    rng = np.random.default_rng(13)
    for (S, D, N, G, k, d, Dout, bias) in [(6, 5, 4, 2, 1, 3, 4, False), (9, 7, 8, 2, 3, 4, 5, True),
                                           (5, 4, 6, 3, 2, 2, 3, False), (7, 6, 8, 1, 5, 8, 2, True),
                                           (4, 3, 4, 4, 1, 2, 2, False)]:
        M = N // G
        x = rng.standard_normal((S, D))
        w_r = rng.standard_normal((G * M, D))
        b_r = rng.standard_normal(G * M) if bias else None
        if not bias and M > 1:  # plant exact router ties: expert 1 copies expert 0
            for g in range(G):
                w_r[g * M + 1] = w_r[g * M]
        Q, K, V = _rand_qkv(rng, 1, S, N, G, d)
        W_O = rng.standard_normal(((G * k + 2) * d, Dout))
        out = O.layer(x, w_r, Q, K, V, W_O, G, k, b_r)
        bf = bruteforce.layer(x.tolist(), w_r.tolist(), Q[0].tolist(), K[0].tolist(), V[0].tolist(),
                              W_O.tolist(), G, k, None if b_r is None else b_r.tolist())
        assert out["idx"].reshape(S, G, k).tolist() == bf["idx"], "brute-force selection"
        _close(out["w"].reshape(S, G, k), bf["w"], 1e-12, "brute-force weights")
        A = O.assemble(out["O_r"].reshape(S, G, k, d), out["w"], out["O_s"].reshape(S, d))
        _close(A, bf["A"], 1e-12, "brute-force slot vectors")
        _close(out["y"], bf["y"], 1e-11, "brute-force y")


def pin_list_invariants(O):
    """|K_g| = k, sum w = 1, each (b,g) list holds k*S entries, lists strictly
    ascending, every token in exactly k lists per group."""
    rng = np.random.default_rng(14)
    B, S, G, M, k, D = 2, 37, 3, 4, 2, 8
    x = rng.standard_normal((B * S, D))
    w_r = rng.standard_normal((G * M, D))
    z, p, idx, w = O.route(x, w_r, G, M, k)
    assert idx.shape == (B * S, G, k)
    assert np.all(np.diff(idx, axis=-1) > 0), "selected experts distinct and ascending"
    _close(w.sum(-1), np.ones((B * S, G)), 1e-14, "sum of renormalised weights")
    # the selection is the top-k of p
    thr = np.sort(p, -1)[..., M - k][..., None]
    assert np.all(np.take_along_axis(p, idx, -1) >= thr)
    off, tok = O.build_lists(idx.reshape(B, S, G, k), M)
    for b in range(B):
        for g in range(G):
            assert off[b, g, 0] == 0 and off[b, g, M] == k * S
            seen = np.zeros(S, int)
            for m in range(M):
                lst = tok[b, g, off[b, g, m]:off[b, g, m + 1]]
                assert np.all(np.diff(lst) > 0)
                for t in lst:
                    assert m in idx.reshape(B, S, G, k)[b, t, g]
                seen[lst] += 1
            assert np.all(seen == k)


def pin_causality_and_compaction(O):
    """Outputs of token i do not depend on tokens after i, nor on how the
    other tokens were routed; decode at position p equals prefill row p."""
    rng = np.random.default_rng(15)
    B, S, N, G, d, k = 1, 12, 8, 2, 4, 2
    M = N // G
    Q, K, V = _rand_qkv(rng, B, S, N, G, d)
    idx = np.sort(rng.permuted(np.tile(np.arange(M), (B, S, G, 1)), axis=-1)[..., :k], -1)
    O_r, O_s = O.prefill(Q, K, V, idx, M)
    i = 6
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    Q2[:, i + 1:] += 1.0
    K2[:, :, i + 1:] -= 2.0
    V2[:, :, i + 1:] *= 3.0
    # reroute every other token (a fresh valid selection), keep token i's
    idx2 = np.sort(rng.permuted(np.tile(np.arange(M), (B, S, G, 1)), axis=-1)[..., :k], -1)
    idx2[:, i] = idx[:, i]
    assert np.any(idx2 != idx)
    O_r2, O_s2 = O.prefill(Q2, K2, V2, idx2, M)
    _close(O_r2[:, i], O_r[:, i], 1e-13, "causality / compaction independence")
    _close(O_s2[:, i], O_s[:, i], 1e-13, "shared head causality")
    # decode of the token at position p against the first p+1 keys
    for p in (0, 5, S - 1):
        Od, Osd = O.decode(Q[:, p:p + 1], K, V, np.array([p + 1]), idx[:, p:p + 1], M)
        _close(Od[:, 0], O_r[:, p], 1e-13, "decode == prefill row")
        _close(Osd[:, 0], O_s[:, p], 1e-13, "decode shared == prefill row")
    # q_len = 2 decode rows equal prefill rows p-1, p
    Od, _ = O.decode(Q[:, 8:10], K, V, np.array([10]), idx[:, 8:10], M)
    _close(Od, O_r[:, 8:10], 1e-13, "multi-token decode == prefill rows")


def pin_boundary_matrix(O):
    """q_len in {1,2}, kv_len in {7,17}, G in {1,2,H} with H = 8, distinct KV
    heads: decode equals the brute-force attention of the visible keys; an
    unsupported N/G is rejected."""
    rng = np.random.default_rng(16)
    H, d = 8, 4
    for G in (1, 2, H):
        M = H // G
        for L in (1, 2):
            for n in (7, 17):
                q = rng.standard_normal((1, L, H + 1, d))
                K = rng.standard_normal((1, G, 20, d))
                V = rng.standard_normal((1, G, 20, d)) + 10.0 * np.arange(G)[None, :, None, None]
                idx = np.broadcast_to(np.arange(M), (1, L, G, M)).copy()
                O_r, O_s = O.decode(q, K, V, np.array([n]), idx, M)
                for t in range(L):
                    pos = n - L + t
                    for h in range(H):
                        g = h // M
                        ref = bruteforce.attend(q[0, t, h].tolist(), K[0, g].tolist(),
                                                V[0, g].tolist(), pos + 1)
                        _close(O_r[0, t, g, h % M], ref, 1e-12, f"boundary G={G} L={L} n={n}")
                    ref = bruteforce.attend(q[0, t, H].tolist(), K[0, 0].tolist(), V[0, 0].tolist(), pos + 1)
                    _close(O_s[0, t], ref, 1e-12, "boundary shared")
    for bad in [(8, 3, 1), (8, 0, 1), (8, 2, 0), (8, 2, 5)]:
        try:
            O.check_dims(*bad)
        except ValueError:
            continue
        raise AssertionError(f"unsupported configuration {bad} was not rejected")


def pin_flop_count(O):
    """Visible (row, key) pairs of the causal prefill by direct count."""
    for (B, S, G, k, d) in [(1, 5, 2, 1, 4), (3, 11, 4, 2, 8)]:
        pairs = B * (G * k + 1) * sum(i + 1 for i in range(S))
        assert O.prefill_flops(B, S, G, k, d) == 4 * d * pairs


def _one_token_variant(O, Q, K, V, G, k, z, mode):
    """The oracle's layer for one token with a given slot layout: the slot
    weights come from slot_weights (the router's p or w, as the layout
    says), the slot vector from assemble."""
    H1, d = Q.shape
    M = (H1 - 1) // G
    p, idx, w = O.route_select(np.asarray(z, dtype=np.float64)[None], k)
    Q4 = np.asarray(Q, dtype=np.float64)[None, None]
    K4 = np.asarray(K, dtype=np.float64)[None, :, None, :]
    V4 = np.asarray(V, dtype=np.float64)[None, :, None, :]
    O_r, O_s = O.prefill(Q4, K4, V4, idx.reshape(1, 1, G, k), M)
    sw = O.slot_weights(p, idx, w, mode)
    return O.assemble(O_r.reshape(1, G, k, d), sw, O_s.reshape(1, d), mode).reshape(-1)


def pin_ablation_slot_variants(O):
    """The two ablation layouts of the review's Table 2 (section 四), on the
    GQA worked example with a zero router (p = 1/2 for both experts):
    hard concatenation only is A = O alone, k=2 -> [1,0,1,0,0,1,0,1] and
    k=1 (tie -> expert 0) -> [1,0,0,1]; weighted concatenation without the
    renormalised slot scales each hard slot by the router probability p, so
    it is half of that, [.5,0,0,.5] at k=1. Renormalised weights would be
    1 at k=1 and make the two rows coincide; the table scores them
    differently. Neither layout carries the shared head (a NaN shared output
    must not reach A) or the obar slot."""
    g = _golden("gqa_worked_example.json")
    Q = np.vstack([np.array(g["Q"], float), [[0.3, -0.7]]])
    K, V = np.array(g["K"], float), np.array(g["V"], float)
    z0 = np.zeros((2, 2))
    _close(_one_token_variant(O, Q, K, V, 2, 2, z0, "hard"), g["concat"], what="hard, k=2")
    _close(_one_token_variant(O, Q, K, V, 2, 1, z0, "hard"), [1, 0, 0, 1], what="hard, k=1")
    _close(_one_token_variant(O, Q, K, V, 2, 2, z0, "weighted"), 0.5 * np.array(g["concat"], float),
           what="weighted, k=2")
    A_w1 = _one_token_variant(O, Q, K, V, 2, 1, z0, "weighted")
    _close(A_w1, [0.5, 0, 0, 0.5], what="weighted, k=1")
    # the two rows must differ at k = 1 whenever p < 1
    assert np.max(np.abs(A_w1 - _one_token_variant(O, Q, K, V, 2, 1, z0, "hard"))) >= 0.5, \
        "the weighted and hard ablation rows coincide at k = 1"
    # the slot weights in closed form: logits (ln 3, 0) give p = (3/4, 1/4)
    p, idx, w = O.route_select(np.array([[[math.log(3.0), 0.0]]]), 1)
    _close(O.slot_weights(p, idx, w, "weighted"), [[[0.75]]], 1e-15, "weighted slot weight, k=1")
    _close(O.slot_weights(p, idx, w, "full"), [[[1.0]]], 0.0, "full-layout weight, k=1")
    assert O.slot_weights(p, idx, w, "hard") is None
    # M=4, k=2, logits (ln 4, ln 2, 0, ln 2): p = (4,2,1,2)/9, top-2 {0,1}
    # (tie between 1 and 3 -> 1); slot weights (4/9, 2/9), renormalised (2/3, 1/3)
    p, idx, w = O.route_select(np.log(np.array([[[4.0, 2.0, 1.0, 2.0]]])), 2)
    _close(O.slot_weights(p, idx, w, "weighted"), [[[4 / 9, 2 / 9]]], 1e-15, "weighted slot weights, k=2")
    _close(O.slot_weights(p, idx, w, "full"), [[[2 / 3, 1 / 3]]], 1e-15, "full-layout weights, k=2")
    # layout on integer values: slot (g, j) at columns (g*k+j)*d, exact
    O_r = np.arange(2 * 2 * 2 * 3, dtype=float).reshape(2, 2, 2, 3)  # T=2, G=2, k=2, d=3
    sw = np.array([[[0.25, 0.75], [0.5, 0.5]], [[1.0, 0.0], [0.125, 0.875]]])
    O_s = np.full((2, 3), np.nan)
    A_h = O.assemble(O_r, sw, O_s, "hard")
    A_w = O.assemble(O_r, sw, O_s, "weighted")
    assert A_h.shape == (2, 12) and A_w.shape == (2, 12), "ablation layouts hold the hard slots only"
    for t in range(2):
        for gg in range(2):
            for j in range(2):
                c = (gg * 2 + j) * 3
                _close(A_h[t, c:c + 3], O_r[t, gg, j], 0.0, "hard slot")
                _close(A_w[t, c:c + 3], sw[t, gg, j] * O_r[t, gg, j], 0.0, "weighted slot")
    assert O.slot_rows(2, 2, 3, "full") == 18 and O.slot_rows(2, 2, 3, "hard") == 12
    assert O.slot_rows(2, 2, 3, "weighted") == 12


# --------------------------------------------------------------------------
# Backward: analytic gradients against central differences of the forward
# --------------------------------------------------------------------------

def _central(f, x, eps=1e-6):
    """Numerical gradient of the scalar f at x (every element), float64."""
    g = np.zeros_like(x)
    flat, gflat = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + eps
        fp = f()
        flat[i] = old - eps
        fm = f()
        flat[i] = old
        gflat[i] = (fp - fm) / (2 * eps)
    return g


def pin_prefill_bwd_central_differences(O):
    """dQ, dK, dV of the sparse causal prefill against central differences of
    sum(dO_r * O_r) + sum(dO_s * O_s); rows of unselected heads get zero."""
    rng = np.random.default_rng(21)
    B, S, N, G, k, d = 1, 5, 4, 2, 1, 3
    M = N // G
    Q = rng.standard_normal((B, S, N + 1, d))
    K = rng.standard_normal((B, G, S, d))
    V = rng.standard_normal((B, G, S, d))
    idx = _random_idx(rng, B, S, G, M, k)
    dO_r = rng.standard_normal((B, S, G, k, d))
    dO_s = rng.standard_normal((B, S, d))

    def loss():
        o_r, o_s = O.prefill(Q, K, V, idx, M)
        return float(np.sum(dO_r * o_r) + np.sum(dO_s * o_s))

    dQ, dK, dV = O.prefill_bwd(Q, K, V, idx, M, dO_r, dO_s)
    _close(dQ, _central(loss, Q), 1e-6, "dQ")
    _close(dK, _central(loss, K), 1e-6, "dK")
    _close(dV, _central(loss, V), 1e-6, "dV")


def pin_prefill_bwd_rows_central_differences(O):
    """prefill_bwd with positions: the gradients of the loss taken over those
    rows alone (sum over them of dO_r * O_r + dO_s * O_s), against central
    differences of that loss; dQ comes back for those rows only."""
    rng = np.random.default_rng(24)
    B, S, N, G, k, d = 2, 7, 6, 3, 1, 3
    M = N // G
    Q = rng.standard_normal((B, S, N + 1, d))
    K = rng.standard_normal((B, G, S, d))
    V = rng.standard_normal((B, G, S, d))
    idx = _random_idx(rng, B, S, G, M, k)
    dO_r = rng.standard_normal((B, S, G, k, d))
    dO_s = rng.standard_normal((B, S, d))
    for pos in (np.array([1, 4, 5]), np.array([6]), np.arange(3, S)):

        def loss():
            o_r, o_s = O.prefill(Q, K, V, idx, M, positions=pos)
            return float(np.sum(dO_r[:, pos] * o_r) + np.sum(dO_s[:, pos] * o_s))

        dQ, dK, dV = O.prefill_bwd(Q, K, V, idx, M, dO_r, dO_s, positions=pos)
        _close(dQ, _central(loss, Q)[:, pos], 1e-6, f"dQ rows {pos}")
        _close(dK, _central(loss, K), 1e-6, f"dK rows {pos}")
        _close(dV, _central(loss, V), 1e-6, f"dV rows {pos}")


def pin_single_key_backward(O):
    """One visible key: o = v_0 whatever q is, so dq = 0, dk_0 = 0 and
    dv_0 = dO (closed form)."""
    rng = np.random.default_rng(22)
    q = rng.standard_normal((1, 4))
    K = rng.standard_normal((3, 4))
    V = rng.standard_normal((3, 4))
    dO = rng.standard_normal((1, 4))
    dq, dK, dV = O.attend_rows_bwd(q, np.array([0]), K, V, dO)
    _close(dq, np.zeros((1, 4)), 1e-12, "single key dq")
    _close(dK, np.zeros((3, 4)), 1e-12, "single key dK")
    _close(dV[0], dO[0], 1e-12, "single key dV")
    _close(dV[1:], np.zeros((2, 4)), 1e-12, "invisible keys dV")


def pin_lse_closed_forms(O):
    """Row log-sum-exp: at position 0 only key 0 is visible, so lse =
    q.k_0/sqrt(d); with every key equal, lse_i = q.k/sqrt(d) + ln(i + 1).
    Per-head queries differ, so a wrong head or KV head shows up."""
    rng = np.random.default_rng(31)
    B, S, G, M, k, d = 2, 6, 2, 3, 2, 4
    N = G * M
    Q = rng.standard_normal((B, S, N + 1, d))
    K = rng.standard_normal((B, G, S, d))
    idx = np.sort(np.stack([rng.permutation(M)[:k] for _ in range(B * S * G)]).reshape(B, S, G, k), axis=-1)
    lse_r, lse_s = O.prefill_lse(Q, K, idx, M)
    for b in range(B):
        for g in range(G):
            for j in range(k):
                h = g * M + idx[b, 0, g, j]
                _close(lse_r[b, 0, g, j], Q[b, 0, h] @ K[b, g, 0] / 2.0, 1e-12, "lse at position 0")
        _close(lse_s[b, 0], Q[b, 0, N] @ K[b, 0, 0] / 2.0, 1e-12, "shared lse at position 0")
    Kc = np.repeat(K[:, :, :1], S, axis=2)  # every key equal to key 0
    lse_r, lse_s = O.prefill_lse(Q, Kc, idx, M)
    ln = np.log(np.arange(1, S + 1))
    for b in range(B):
        _close(lse_s[b], Q[b, :, N] @ K[b, 0, 0] / 2.0 + ln, 1e-12, "shared lse, equal keys")
        for g in range(G):
            for j in range(k):
                h = g * M + idx[b, :, g, j]
                sc = np.einsum("sd,d->s", Q[b, np.arange(S), h], K[b, g, 0]) / 2.0
                _close(lse_r[b, :, g, j], sc + ln, 1e-12, "lse, equal keys")


def pin_lse_positions_closed_form(O):
    """prefill_lse at chosen positions, every key equal: lse_i = q_i.k/sqrt(d)
    + ln(i + 1) with the query of the row's own head (closed form)."""
    rng = np.random.default_rng(32)
    B, S, G, M, k, d = 1, 9, 2, 2, 1, 4
    N = G * M
    Q = rng.standard_normal((B, S, N + 1, d))
    K = np.repeat(rng.standard_normal((B, G, 1, d)), S, axis=2)
    idx = rng.integers(0, M, (B, S, G, k))
    pos = np.array([0, 3, 8])
    lse_r, lse_s = O.prefill_lse(Q, K, idx, M, positions=pos)
    ln = np.log(pos + 1.0)
    _close(lse_s[0], Q[0, pos, N] @ K[0, 0, 0] / 2.0 + ln, 1e-12, "shared lse at positions")
    for g in range(G):
        h = g * M + idx[0, pos, g, 0]
        _close(lse_r[0, :, g, 0], np.einsum("pd,d->p", Q[0, pos, h], K[0, g, 0]) / 2.0 + ln, 1e-12,
               "lse at positions")


def pin_out_proj_bwd_central_differences(O):
    """dO_r, dw, dO_s, dW_O of y = A W_O (all three slot layouts) against
    central differences of sum(dy * y). In the ablation layouts the shared
    head does not reach y, so its gradient is 0; in the hard one the slot
    weights do not either."""
    rng = np.random.default_rng(23)
    T, G, k, d, D = 3, 2, 2, 2, 5
    O_r = rng.standard_normal((T, G, k, d))
    w = rng.random((T, G, k))
    O_s = rng.standard_normal((T, d))
    dy = rng.standard_normal((T, D))
    for mode, rows in (("full", (G * k + 2) * d), ("hard", G * k * d), ("weighted", G * k * d)):
        W_O = rng.standard_normal((rows, D))

        def loss():
            return float(np.sum(dy * O.out_proj(O_r, w, O_s, W_O, mode=mode)))

        dO_r, dw, dO_s, dW_O = O.out_proj_bwd(O_r, w, O_s, W_O, dy, mode=mode)
        _close(dO_r, _central(loss, O_r), 1e-6, f"{mode} dO_r")
        _close(dw, _central(loss, w), 1e-6, f"{mode} dw")
        _close(dO_s, _central(loss, O_s), 1e-6, f"{mode} dO_s")
        _close(dW_O, _central(loss, W_O), 1e-6, f"{mode} dW_O")


def pin_route_bwd_central_differences(O):
    """dW_r, db_r, dx of the renormalised top-k weights against central
    differences of sum(dw * w(x, W_r, b_r)); the logits are far apart, so
    the perturbations never change the selection."""
    rng = np.random.default_rng(24)
    T, D, G, M, k = 4, 6, 2, 4, 2
    x = rng.standard_normal((T, D))
    w_r = rng.standard_normal((G * M, D))
    b_r = rng.standard_normal(G * M) * 3.0
    dw = rng.standard_normal((T, G, k))

    def loss():
        _, _, _, ww = O.route(x, w_r, G, M, k, b_r)
        return float(np.sum(dw * ww))

    z, _, idx, _ = O.route(x, w_r, G, M, k, b_r)
    dz, dW_r, db_r, dx = O.route_bwd(x, w_r, z, idx, dw, G, M)
    _close(dW_r, _central(loss, w_r), 1e-6, "dW_r")
    _close(db_r, _central(loss, b_r), 1e-6, "db_r")
    _close(dx, _central(loss, x), 1e-6, "dx")


def pin_route_bwd_probability_weights(O):
    """route_bwd with wrt="p" (the weighted-concatenation ablation, whose
    slot weights are the selected router probabilities): dW_r, db_r, dx
    against central differences of sum(dw * p_sel(x, W_r, b_r)), and the
    closed form at M = 2, k = 1: d p_0 / d z_0 = p_0 p_1."""
    rng = np.random.default_rng(26)
    T, D, G, M, k = 4, 6, 2, 4, 2
    x = rng.standard_normal((T, D))
    w_r = rng.standard_normal((G * M, D))
    b_r = rng.standard_normal(G * M) * 3.0
    dw = rng.standard_normal((T, G, k))

    def loss():
        _, p, idx_, _ = O.route(x, w_r, G, M, k, b_r)
        return float(np.sum(dw * np.take_along_axis(p, idx_, -1)))

    z, _, idx, _ = O.route(x, w_r, G, M, k, b_r)
    dz, dW_r, db_r, dx = O.route_bwd(x, w_r, z, idx, dw, G, M, wrt="p")
    _close(dW_r, _central(loss, w_r), 1e-6, "dW_r (wrt p)")
    _close(db_r, _central(loss, b_r), 1e-6, "db_r (wrt p)")
    _close(dx, _central(loss, x), 1e-6, "dx (wrt p)")
    # M = 2, k = 1, logits (ln 3, 0): p = (3/4, 1/4), expert 0 selected;
    # dz = dw * (p0 p1, -p0 p1) = dw * (3/16, -3/16)
    z1 = np.array([[[math.log(3.0), 0.0]]])
    dz1, _, _, _ = O.route_bwd(np.zeros((1, 1)), np.zeros((2, 1)), z1, np.array([[[0]]]),
                               np.array([[[2.0]]]), 1, 2, wrt="p")
    _close(dz1, [[[0.375, -0.375]]], 1e-15, "dz closed form (wrt p)")


def pin_load_balance_closed_forms(O):
    """Balance loss: equal logits with every expert chosen equally often
    give exactly coef; every token on expert 0 with p_0 -> 1 gives coef*M;
    a router with p uniform but all tokens on one expert gives coef (f . P
    = 1/M)."""
    T, G, M, k, coef = 8, 2, 4, 1, 0.01
    idx = np.tile(np.arange(T) % M, (G, 1)).T.reshape(T, G, k)
    _close(O.load_balance_loss(np.zeros((T, G, M)), idx, M, coef), coef, 1e-15, "balanced")
    z = np.zeros((T, G, M))
    z[..., 0] = 60.0
    one = np.zeros((T, G, k), dtype=np.int64)
    _close(O.load_balance_loss(z, one, M, coef), coef * M, 1e-12, "collapsed")
    _close(O.load_balance_loss(np.zeros((T, G, M)), one, M, coef), coef, 1e-15, "uniform p, one expert")
    idx2 = np.stack([np.sort(np.random.default_rng(t).permutation(M)[:2]) for t in range(T * G)]).reshape(T, G, 2)
    _close(O.load_balance_loss(np.zeros((T, G, M)), idx2, M, coef), coef, 1e-15, "uniform p, k = 2")


def pin_route_bwd_balance_loss_central_differences(O):
    """dz of the balance loss (route_bwd with dw = 0) against central
    differences in the logits with the selection held fixed, and dz of
    route_bwd (dw and balance loss together) against differences of their
    sum."""
    rng = np.random.default_rng(25)
    T, D, G, M, k, coef = 5, 6, 2, 4, 2, 0.3
    x = rng.standard_normal((T, D))
    w_r = rng.standard_normal((G * M, D))
    z = rng.standard_normal((T, G, M))
    idx = np.sort(np.argsort(-z, axis=-1)[..., :k], axis=-1)
    dw = rng.standard_normal((T, G, k))

    def loss():
        p = O.softmax(z, axis=-1)
        ps = np.take_along_axis(p, idx, -1)
        ww = ps / ps.sum(-1, keepdims=True)
        return float(np.sum(dw * ww)) + O.load_balance_loss(z, idx, M, coef)

    dz0, _, _, _ = O.route_bwd(x, w_r, z, idx, np.zeros_like(dw), G, M, aux_coef=coef)

    def aux_only():
        return O.load_balance_loss(z, idx, M, coef)

    _close(dz0, _central(aux_only, z), 1e-8, "balance-loss dz")
    dz, _, _, _ = O.route_bwd(x, w_r, z, idx, dw, G, M, aux_coef=coef)
    _close(dz, _central(loss, z), 1e-7, "dz with balance loss")


# --------------------------------------------------------------------------
# Projections: token-compacted Q, dense K/V, decode append
# --------------------------------------------------------------------------

def _selector_weights(N, G, d, D):
    """W_Q block h copies coordinates h*d..h*d+d-1 of x (the shared block N
    included); W_K block g copies the G*d coordinates after those, and W_V
    block g twice the G*d coordinates after the keys'."""
    W_Q = np.zeros(((N + 1) * d, D))
    W_K = np.zeros((G * d, D))
    W_V = np.zeros((G * d, D))
    for r in range((N + 1) * d):
        W_Q[r, r] = 1.0
    for r in range(G * d):
        W_K[r, (N + 1) * d + r] = 1.0
        W_V[r, (N + 1 + G) * d + r] = 2.0
    return W_Q, W_K, W_V


def _random_idx(rng, B, S, G, M, k):
    return np.sort(rng.permuted(np.tile(np.arange(M), (B, S, G, 1)), axis=-1)[..., :k], -1)


def pin_projection_closed_form(O):
    """With coordinate-selecting weights every projected row is a slice of x:
    the selected heads' and the shared head's query rows, every key and value
    row; the rows of heads a token did not select are not computed."""
    rng = np.random.default_rng(11)
    B, S, N, G, k, d = 2, 7, 6, 2, 2, 3
    M = N // G
    D = (N + 1 + 2 * G) * d + 5
    x = rng.standard_normal((B, S, D))
    W_Q, W_K, W_V = _selector_weights(N, G, d, D)
    idx = _random_idx(rng, B, S, G, M, k)
    Q, K, V = O.project(x, W_Q, W_K, W_V, idx, N, G)
    assert Q.shape == (B, S, N + 1, d) and K.shape == (B, G, S, d) and V.shape == (B, G, S, d)
    kb, vb = (N + 1) * d, (N + 1 + G) * d
    for b in range(B):
        for i in range(S):
            chosen = {g * M + int(m) for g in range(G) for m in idx[b, i, g]} | {N}
            for h in range(N + 1):
                if h in chosen:
                    _close(Q[b, i, h], x[b, i, h * d:(h + 1) * d], what=f"q of head {h}")
                else:
                    assert np.all(np.isnan(Q[b, i, h])), f"unselected head {h} of token {i} computed"
            for g in range(G):
                _close(K[b, g, i], x[b, i, kb + g * d:kb + (g + 1) * d], what=f"k of group {g}")
                _close(V[b, g, i], 2 * x[b, i, vb + g * d:vb + (g + 1) * d], what=f"v of group {g}")


def pin_projection_dense_reduction(O):
    """k = M selects every head, so the compacted projection equals the dense
    linear layer torch.nn.functional.linear(x, W) = x W^T: all N+1 query
    heads, and K and V laid out [B, G, S, d]."""
    rng = np.random.default_rng(12)
    B, S, N, G, d, D = 2, 9, 8, 2, 4, 24
    M = N // G
    x = rng.standard_normal((B, S, D))
    W_Q, W_K, W_V = (rng.standard_normal((r, D)) for r in ((N + 1) * d, G * d, G * d))
    idx = np.broadcast_to(np.arange(M), (B, S, G, M)).copy()
    Q, K, V = O.project(x, W_Q, W_K, W_V, idx, N, G)

    def lin(w):
        return torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()

    _close(Q, lin(W_Q).reshape(B, S, N + 1, d), 1e-10, "dense Q")
    _close(K, lin(W_K).reshape(B, S, G, d).transpose(0, 2, 1, 3), 1e-10, "dense K")
    _close(V, lin(W_V).reshape(B, S, G, d).transpose(0, 2, 1, 3), 1e-10, "dense V")


def pin_projection_row_count(O):
    """Every token computes exactly G*k routed query rows plus the shared one:
    9 of 17 heads at N = 16, G = 8, k = 1 ([GQE-review] §二: 8 routed heads
    plus the shared head per token). The FLOP count is 2*D per computed
    output value."""
    rng = np.random.default_rng(13)
    B, S, N, G, k, d, D = 2, 6, 16, 8, 1, 2, 8
    x = rng.standard_normal((B, S, D))
    W_Q, W_K, W_V = (rng.standard_normal((r, D)) for r in ((N + 1) * d, G * d, G * d))
    idx = _random_idx(rng, B, S, G, N // G, k)
    Q, K, V = O.project(x, W_Q, W_K, W_V, idx, N, G)
    computed = ~np.all(np.isnan(Q), axis=-1)  # [B, S, N+1]
    assert np.all(computed.sum(axis=-1) == 9) and np.all(computed[..., N])
    n_out = int(computed.sum()) * d + K.size + V.size
    assert O.project_flops(B * S, D, G, k, d) == 2 * D * n_out


def pin_decode_append(O):
    """The new tokens' keys and values land in cache rows kv_len-q_len+t and
    nowhere else; their queries are the prefill projection of the same
    tokens."""
    rng = np.random.default_rng(14)
    B, L, N, G, k, d, Smax = 3, 2, 4, 2, 1, 2, 9
    D = (N + 1 + 2 * G) * d
    x = rng.standard_normal((B, L, D))
    W_Q, W_K, W_V = _selector_weights(N, G, d, D)
    idx = _random_idx(rng, B, L, G, N // G, k)
    kv_len = np.array([2, 5, 9])
    Kc0 = rng.standard_normal((B, G, Smax, d))
    Vc0 = rng.standard_normal((B, G, Smax, d))
    Q, Kc, Vc = O.project_decode(x, W_Q, W_K, W_V, idx, N, G, kv_len, Kc0, Vc0)
    kb, vb = (N + 1) * d, (N + 1 + G) * d
    for b in range(B):
        n = int(kv_len[b])
        for j in range(Smax):
            t = j - (n - L)
            if 0 <= t < L:
                for g in range(G):
                    _close(Kc[b, g, j], x[b, t, kb + g * d:kb + (g + 1) * d], what="appended k")
                    _close(Vc[b, g, j], 2 * x[b, t, vb + g * d:vb + (g + 1) * d], what="appended v")
            else:
                assert np.array_equal(Kc[b, :, j], Kc0[b, :, j]), f"cache row {j} of sequence {b} changed"
                assert np.array_equal(Vc[b, :, j], Vc0[b, :, j]), f"cache row {j} of sequence {b} changed"
    Qp, _, _ = O.project(x, W_Q, W_K, W_V, idx, N, G)
    assert np.array_equal(np.isnan(Q), np.isnan(Qp))
    _close(np.nan_to_num(Q), np.nan_to_num(Qp), what="decode queries")


ALL_PINS = [v for kname, v in sorted(globals().items()) if kname.startswith("pin_")]
