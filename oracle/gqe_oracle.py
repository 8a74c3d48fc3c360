"""Plain CPU oracle for the Grouped Query Experts (GQE) attention layer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module. The GPU library never imports, calls or
links it, and it shares no code with the GPU library: it is NumPy only, in
float64 by default, written as the plain definition of each step.

Sources (cited by page title and section):

[GQE-review]  "论文综述：分组查询专家——在 GQA 自注意力上引入混合专家"
              (paper.oopus.info), §二 核心方法与创新: the router equation
              p_{i,g} = softmax(r_g(x_i)), the TopK equation, the three output
              parts, the renormalised weight w_{i,g,m}, the weighted sum
              ō_i and the output y_i = Concat(O_i, ō_i, s(x_i)) W_O.
[GQE-summary] "Grouped Query Experts: Mixture-of-Experts on GQA Self-Attention"
              (1kpapers.com), In brief: k experts per group, dense KV heads,
              9 of 16 query-attention computations.
[GQA-zone]    "AI 大模型之 GQA" (zone.ci): §4.1 KV-byte formula, §4.3 the
              logical broadcast of KV heads, §技术深化 "分组不是把查询头合并"
              (head i reads KV head floor(i/(H/G)); additive mask; absolute
              query position), §工程实操 non-square causal mask.
[MQA-GQA-171] "MQA、GQA、稀疏/滑动窗口注意力及混合范式" (171host.com): the
              GQA and MQA numeric examples and the KV-cache byte examples.

Readings where the pages are silent (each is listed in the design notes):
  * r_g is affine: z = x W_r[g]^T (+ optional bias b_r[g]); no other form is
    given.
  * TopK keeps the k largest scores, ties going to the lower expert index;
    the selected indices are stored in ascending order. Selecting on the
    logits z gives the same set as selecting on p, because softmax is strictly
    increasing in z within one group.
  * The hard slots of one group are laid out in ascending expert index; the
    groups are laid out g = 0..G-1.
  * ō_i sums over every group g and every selected m (one d-vector).
  * The shared head is query column block N and reads KV head 0, causally,
    with scale 1/sqrt(d) and no routing weight.
  * W_O has shape ((G*k + 2) * d, D_out), no bias.
  * The two ablation rows of [GQE-review] §四 Table 2 keep only the hard
    slots: "hard" plain, "weighted" scaled by the router probabilities p
    (not renormalised); neither has ō or the shared head (assemble).
  * A key j is visible to a query at absolute position p iff j <= p.

parity pinned: every function here is checked against values and identities
fixed by the pages or by mathematics in the CPU tests (worked examples,
closed forms, reductions to dense GQA/MHA/MQA, repeat-KV equivalence, brute
force on tiny inputs).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "softmax", "topk_select", "route_logits", "route_select", "route",
    "build_lists", "attend_rows", "prefill", "decode", "assemble", "out_proj",
    "layer", "kv_bytes", "prefill_flops", "check_dims", "project",
    "project_decode", "project_flops", "attend_rows_bwd", "prefill_bwd",
    "out_proj_bwd", "route_bwd", "lse_rows", "prefill_lse", "load_balance_loss",
    "slot_weights", "slot_rows",
]


def check_dims(N: int, G: int, k: int) -> int:
    """Reject unsupported head configurations; return M = N/G.

    [GQA-zone] §4.4 and §工程实操 (扩展验证组合): the group count must divide the
    query-head count, and unsupported H/G combinations are rejected explicitly,
    never mapped silently.
    """
    if G <= 0 or N <= 0 or N % G != 0:
        raise ValueError(f"unsupported head configuration N={N}, G={G}: G must divide N")
    M = N // G
    if not 1 <= k <= M:
        raise ValueError(f"unsupported top-k k={k} for M={M} experts per group")
    return M


def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    """softmax with the usual max subtraction (exact in real arithmetic)."""
    z = np.asarray(z, dtype=np.float64)
    zmax = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - zmax)
    return e / np.sum(e, axis=axis, keepdims=True)


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """TopK over the last axis: indices of the k largest scores, ascending.

    [GQE-review] §二 路由器, the TopK equation K_g(x_i) = TopK_m(p_{i,g,m}, k).
    Ties go to the lower index (a stable sort of the negated scores keeps
    equal scores in index order).
    """
    order = np.argsort(-np.asarray(scores), axis=-1, kind="stable")
    return np.sort(order[..., :k], axis=-1).astype(np.int64)


def route_logits(x: np.ndarray, w_r: np.ndarray, G: int, M: int,
                 b_r: np.ndarray | None = None) -> np.ndarray:
    """Router scores z_{i,g} = r_g(x_i) in R^M for every token and group.

    [GQE-review] §二 路由器: one router r_g per GQA group scores the group's M
    query-head experts. x: [T, D]; w_r: [G*M, D]; b_r: [G*M] or None.
    Returns z [T, G, M].
    """
    z = np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T
    if b_r is not None:
        z = z + np.asarray(b_r, dtype=np.float64)[None, :]
    return z.reshape(z.shape[0], G, M)


def route_select(z: np.ndarray, k: int):
    """Softmax, TopK and renormalised weights from router scores z [T, G, M].

    [GQE-review] §二: p = softmax(z); K_g = TopK(p, k);
    w_{i,g,m} = p_{i,g,m} / sum_{m' in K_g} p_{i,g,m'}.
    Returns (p [T,G,M], idx [T,G,k] ascending, w [T,G,k]).
    """
    p = softmax(z, axis=-1)
    idx = topk_select(z, k)
    p_sel = np.take_along_axis(p, idx, axis=-1)
    w = p_sel / np.sum(p_sel, axis=-1, keepdims=True)
    return p, idx, w


def route(x, w_r, G: int, M: int, k: int, b_r=None):
    """Full router: returns (z, p, idx, w) as route_logits + route_select."""
    z = route_logits(x, w_r, G, M, b_r)
    p, idx, w = route_select(z, k)
    return z, p, idx, w


def build_lists(idx: np.ndarray, M: int):
    """Per-(sequence, group, expert) token lists.

    idx: [B, S, G, k] selected experts. For each (b, g) the list of expert m
    holds, in ascending order, the positions of the tokens whose selection in
    group g contains m; the lists of m = 0..M-1 are stored one after another.
    Returns (list_off [B, G, M+1], list_tok [B, G, k*S]) with list m occupying
    list_tok[b, g, list_off[b,g,m]:list_off[b,g,m+1]].
    """
    B, S, G, k = idx.shape
    off = np.zeros((B, G, M + 1), dtype=np.int64)
    tok = np.zeros((B, G, k * S), dtype=np.int64)
    for b in range(B):
        for g in range(G):
            pos = 0
            for m in range(M):
                rows = np.nonzero(np.any(idx[b, :, g, :] == m, axis=-1))[0]
                off[b, g, m] = pos
                tok[b, g, pos:pos + rows.size] = rows
                pos += rows.size
            off[b, g, M] = pos
    return off, tok


def attend_rows(q: np.ndarray, pos: np.ndarray, K: np.ndarray, V: np.ndarray,
                row_chunk: int = 1024) -> np.ndarray:
    """Causal scaled dot-product attention of query rows against one KV head.

    o_r = sum_{j <= pos_r} softmax_j(q_r . k_j / sqrt(d)) v_j.
    [GQA-zone] §技术深化: scores Q K^T / sqrt(d), additive mask (0 where
    visible, -inf where not) decided by the query's absolute position, softmax,
    then V. q: [n, d]; pos: [n] absolute positions; K, V: [S, d].
    """
    q = np.asarray(q, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    n, d = q.shape
    out = np.zeros((n, V.shape[-1]), dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        qr, pr = q[r0:r0 + row_chunk], pos[r0:r0 + row_chunk]
        if qr.shape[0] == 0:
            continue
        L = int(pr.max()) + 1
        s = (qr @ K[:L].T) / np.sqrt(d)
        mask = np.where(np.arange(L)[None, :] <= pr[:, None], 0.0, -np.inf)
        s = s + mask
        s = s - np.max(s, axis=1, keepdims=True)
        e = np.exp(s)
        out[r0:r0 + qr.shape[0]] = (e / np.sum(e, axis=1, keepdims=True)) @ V[:L]
    return out


def prefill(Q, K, V, idx, M: int, positions=None, q_rows_only: bool = False):
    """Sparse-query causal attention for a prefill of S tokens per sequence.

    Q: [B, S, N+1, d] (head N is the shared head); K, V: [B, G, S, d];
    idx: [B, S, G, k] selected experts. For token i, group g and slot j the
    head is h = g*M + idx[b,i,g,j] and it attends KV head g
    ([GQA-zone] §技术深化: query head i reads KV head floor(i/(H/G)));
    only selected heads are computed ([GQE-review] §二, unselected heads are
    skipped). The shared head attends KV head 0 for every token.
    positions: token positions to compute (default: all S). With
    q_rows_only, Q holds just the rows of those positions ([B, P, N+1, d]),
    for sequences whose whole Q would not fit in memory as float64.
    Returns (O_r [B, P, G, k, d], O_s [B, P, d]) for the P positions.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, G, S, d = K.shape
    k = idx.shape[-1]
    N = np.shape(Q)[2] - 1
    check_dims(N, G, k)
    pos = np.arange(S) if positions is None else np.asarray(positions, dtype=np.int64)
    Qp = np.asarray(Q if q_rows_only else np.asarray(Q)[:, pos], dtype=np.float64)  # [B, P, N+1, d]
    rows = np.arange(pos.size)
    O_r = np.zeros((B, pos.size, G, k, d))
    O_s = np.zeros((B, pos.size, d))
    for b in range(B):
        for g in range(G):
            for j in range(k):
                heads = g * M + idx[b, pos, g, j]
                O_r[b, :, g, j] = attend_rows(Qp[b, rows, heads, :], pos, K[b, g], V[b, g])
        O_s[b] = attend_rows(Qp[b, :, N, :], pos, K[b, 0], V[b, 0])
    return O_r, O_s


def lse_rows(q, pos, K):
    """Log of the softmax normaliser of each query row: ln sum_{j <= pos}
    exp(q . k_j / sqrt(d)), the same visible scores as attend_rows
    ([GQA-zone] §技术深化). A training forward keeps it so that the
    backward can rebuild P = exp(s - lse) without the running max.
    q: [n, d]; pos: [n]; K: [S, d]. Returns [n].
    """
    q = np.asarray(q, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    n, d = q.shape
    if n == 0:
        return np.zeros(0)
    L = int(pos.max()) + 1
    sc = (q @ np.asarray(K, dtype=np.float64)[:L].T) / np.sqrt(d)
    sc = np.where(np.arange(L)[None, :] <= pos[:, None], sc, -np.inf)
    top = np.max(sc, axis=1)
    return top + np.log(np.sum(np.exp(sc - top[:, None]), axis=1))


def prefill_lse(Q, K, idx, M: int, positions=None):
    """lse_rows for every row prefill computes: (lse_r [B, P, G, k],
    lse_s [B, P]), same head mapping and shared head as prefill, for the
    P positions given (default: all S)."""
    Q = np.asarray(Q, dtype=np.float64)
    B, S, H1, d = Q.shape
    G = K.shape[1]
    k = idx.shape[-1]
    N = H1 - 1
    check_dims(N, G, k)
    pos = np.arange(S) if positions is None else np.asarray(positions, dtype=np.int64)
    lse_r = np.zeros((B, pos.size, G, k))
    lse_s = np.zeros((B, pos.size))
    for b in range(B):
        for g in range(G):
            for j in range(k):
                heads = g * M + idx[b, pos, g, j]
                lse_r[b, :, g, j] = lse_rows(Q[b, pos, heads, :], pos, K[b, g])
        lse_s[b] = lse_rows(Q[b, pos, N, :], pos, K[b, 0])
    return lse_r, lse_s


def decode(q, K, V, kv_len, idx, M: int, kv_start=None):
    """Sparse-query attention of q_len new tokens per sequence against a cache.

    q: [B, q_len, N+1, d]; K, V: [B, G, S_max, d]; kv_len: [B] valid cache
    length including the new tokens; idx: [B, q_len, G, k].
    New token t of sequence b sits at absolute position kv_len[b]-q_len+t and
    sees keys j <= that position ([GQA-zone] §技术深化 and §工程实操: in decode
    Sq is small and Sk is the full history, so the causal mask must use the
    query's absolute position, not a top-left triangle).
    kv_start: optional [B]; keys j < kv_start[b] are padding and visible to
    no query (visibility = causal and key-valid, [GQA-zone] §工程实操 on
    padding masks).
    Returns (O_r [B, q_len, G, k, d], O_s [B, q_len, d]).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, L, H1, d = q.shape
    G = K.shape[1]
    k = idx.shape[-1]
    N = H1 - 1
    check_dims(N, G, k)
    O_r = np.zeros((B, L, G, k, d))
    O_s = np.zeros((B, L, d))
    for b in range(B):
        n = int(kv_len[b])
        if n < L or n > K.shape[2]:
            raise ValueError("kv_len must satisfy q_len <= kv_len <= S_max")
        s0 = 0 if kv_start is None else int(kv_start[b])
        if s0 < 0 or s0 > n - L:
            raise ValueError("kv_start must satisfy 0 <= kv_start <= kv_len - q_len")
        pos = n - L + np.arange(L) - s0  # positions within the valid keys s0 .. n-1
        for g in range(G):
            for j in range(k):
                heads = g * M + idx[b, :, g, j]
                O_r[b, :, g, j] = attend_rows(q[b, np.arange(L), heads, :], pos,
                                              K[b, g, s0:n], V[b, g, s0:n])
        O_s[b] = attend_rows(q[b, :, N, :], pos, K[b, 0, s0:n], V[b, 0, s0:n])
    return O_r, O_s


def slot_weights(p, idx, w, mode: str = "full"):
    """Per-slot weights [T, G, k] that each slot layout applies to the
    selected heads' outputs.

    "full": the renormalised weights w of the ō slot ([GQE-review] §二, the
    w equation). "weighted": the Table 2 row of [GQE-review] §四 that keeps
    only a weighted concatenation and removes the renormalised slot, so each
    hard slot is scaled by the router's own
    probability p_{i,g,m} (the group softmax over all M experts, not
    renormalised over the selected set). Renormalised weights would be
    exactly 1 at the pages' k = 1 and make this row the hard one, which the
    table's two different scores rule out. "hard": no weights (None).
    p: [T, G, M]; idx: [T, G, k]; w: [T, G, k].
    """
    if mode == "full":
        return np.asarray(w, dtype=np.float64)
    if mode == "weighted":
        return np.take_along_axis(np.asarray(p, dtype=np.float64), np.asarray(idx), axis=-1)
    if mode == "hard":
        return None
    raise ValueError(f"unknown slot mode {mode!r}")


def assemble(O_r, w, O_s, mode: str = "full") -> np.ndarray:
    """Slot vector A_i = Concat(O_i, ō_i, s(x_i)) for every token.

    [GQE-review] §二 输出怎么拼起来: hard-selected slot O_i (the selected heads'
    outputs, concatenated), renormalised weighted-sum slot
    ō_i = sum w_{i,g,m} o_{i,g,m} (summed over all groups), and the shared
    head's output s(x_i).
    The ablation rows of [GQE-review] §四 (Table 2) each keep only one kind
    of concatenation: mode "hard" (hard concatenation only) is A_i = O_i,
    and mode "weighted" (weighted concatenation only, renormalised slot
    removed) is A_i = w ⊙ O_i with w the slot weights of
    slot_weights(..., "weighted"), the router probabilities p. Neither has
    the ō slot or the shared head: each row's label names the one part it
    keeps, the note under the table ties the drops to removing the
    renormalised slot and the shared head / soft signal, and [GQE-summary]
    (In brief) has the ablations lacking both the renormalised slot and the
    shared head.
    O_r: [T, G, k, d]; w: [T, G, k] (mode "full": renormalised weights;
    "weighted": the slot weights; "hard": unused); O_s: [T, d] (unused by the
    ablation modes). Returns [T, (G*k+2)*d] (full) or [T, G*k*d].
    """
    O_r = np.asarray(O_r, dtype=np.float64)
    T, G, k, d = O_r.shape
    if mode == "full":
        w = np.asarray(w, dtype=np.float64)
        shared = np.asarray(O_s, dtype=np.float64)
        hard = O_r.reshape(T, G * k * d)
        obar = np.sum(w[..., None] * O_r, axis=(1, 2))
        return np.concatenate([hard, obar, shared], axis=1)
    if mode == "hard":
        return O_r.reshape(T, G * k * d)
    if mode == "weighted":
        w = np.asarray(w, dtype=np.float64)
        return (w[..., None] * O_r).reshape(T, G * k * d)
    raise ValueError(f"unknown slot mode {mode!r}")


def slot_rows(G: int, k: int, d: int, mode: str = "full") -> int:
    """Rows of W_O for a slot layout: (G*k+2)*d for the full [O, ō, s],
    G*k*d for the ablation layouts (hard slots only)."""
    if mode == "full":
        return (G * k + 2) * d
    if mode in ("hard", "weighted"):
        return G * k * d
    raise ValueError(f"unknown slot mode {mode!r}")


def out_proj(O_r, w, O_s, W_O, mode: str = "full") -> np.ndarray:
    """y_i = Concat(O_i, ō_i, s(x_i)) W_O  ([GQE-review] §二, the y equation),
    or the same product with an ablation variant's slot vector."""
    return assemble(O_r, w, O_s, mode) @ np.asarray(W_O, dtype=np.float64)


def layer(x, w_r, Q, K, V, W_O, G: int, k: int, b_r=None, mode: str = "full"):
    """Whole prefill layer: route, attend, assemble, project. Returns a dict.
    mode picks the slot layout (assemble); the slot weights it uses are
    slot_weights(p, idx, w, mode)."""
    B, S, H1, d = np.asarray(Q).shape
    N = H1 - 1
    M = check_dims(N, G, k)
    z, p, idx, w = route(np.asarray(x).reshape(B * S, -1), w_r, G, M, k, b_r)
    idx4 = idx.reshape(B, S, G, k)
    O_r, O_s = prefill(Q, K, V, idx4, M)
    T = B * S
    sw = slot_weights(p, idx, w, mode)
    y = out_proj(O_r.reshape(T, G, k, d), sw, O_s.reshape(T, d), W_O, mode)
    return dict(z=z, p=p, idx=idx, w=w, sw=sw, O_r=O_r, O_s=O_s, y=y)


def project(x, W_Q, W_K, W_V, idx, N: int, G: int):
    """Query, key and value projections of a prefill, Q compacted to the
    heads that are used.

    [GQE-review] §二: only the selected query heads take part in attention and
    the rest are skipped, so only their query rows are computed; the shared
    head s(x_i) is computed for every token. [GQA-zone] §4.3: queries carry H
    heads and keys/values G heads (stored here as [B, G, S, d]).
    The projections are linear without bias (a reading: the pages give no
    other form): q_{i,h} = W_Q[h] x_i, where W_Q[h] is rows h*d .. h*d+d-1 of
    W_Q and block N is the shared head; k_{i,g} = W_K[g] x_i, v_{i,g} =
    W_V[g] x_i with G blocks of d rows each.
    x: [B, S, D]; W_Q: [(N+1)*d, D]; W_K, W_V: [G*d, D]; idx: [B, S, G, k].
    Returns (Q [B, S, N+1, d], NaN in every row that is not computed,
    K [B, G, S, d], V [B, G, S, d]).
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    B, S, D = x.shape
    M = check_dims(N, G, idx.shape[-1])
    W_Q = np.asarray(W_Q, dtype=np.float64)
    d = W_Q.shape[0] // (N + 1)
    Wq = W_Q.reshape(N + 1, d, D)
    Q = np.full((B, S, N + 1, d), np.nan)
    for h in range(N):
        g, m = divmod(h, M)
        chose = np.any(idx[:, :, g, :] == m, axis=-1)  # [B, S]: tokens whose group g picked m
        Q[chose, h] = x[chose] @ Wq[h].T
    Q[:, :, N] = x @ Wq[N].T
    K = (x @ np.asarray(W_K, dtype=np.float64).T).reshape(B, S, G, d).transpose(0, 2, 1, 3)
    V = (x @ np.asarray(W_V, dtype=np.float64).T).reshape(B, S, G, d).transpose(0, 2, 1, 3)
    return Q, K, V


def project_decode(x, W_Q, W_K, W_V, idx, N: int, G: int, kv_len, K_cache, V_cache):
    """The projections of q_len new tokens per sequence, with their key and
    value rows written into the caches.

    New token t of sequence b sits at absolute position kv_len[b]-q_len+t
    ([GQA-zone] §技术深化: a decode query's absolute position), which is the
    cache row that receives its key and value; no other row changes.
    x: [B, q_len, D]; idx: [B, q_len, G, k]; kv_len: [B];
    K_cache, V_cache: [B, G, S_max, d].
    Returns (Q [B, q_len, N+1, d] with NaN rows as in project, the new K cache,
    the new V cache).
    """
    Q, K, V = project(x, W_Q, W_K, W_V, idx, N, G)
    Kc = np.array(K_cache, dtype=np.float64, copy=True)
    Vc = np.array(V_cache, dtype=np.float64, copy=True)
    L = Q.shape[1]
    for b in range(Q.shape[0]):
        n = int(kv_len[b])
        if n < L or n > Kc.shape[2]:
            raise ValueError("kv_len must satisfy q_len <= kv_len <= S_max")
        Kc[b, :, n - L:n] = K[b]
        Vc[b, :, n - L:n] = V[b]
    return Q, Kc, Vc


def project_flops(T: int, D: int, G: int, k: int, d: int) -> int:
    """Matmul FLOP of the projections: 2*D per output element, with
    (G*k+1)*d query columns (the selected heads and the shared head) and
    2*G*d key/value columns per token."""
    return 2 * T * D * ((G * k + 1) * d + 2 * G * d)


# --------------------------------------------------------------------------
# Backward pass: gradients of the scalar loss sum(dy * y) (the reverse-mode
# derivatives of the functions above, written out)
# --------------------------------------------------------------------------

def attend_rows_bwd(q, pos, K, V, dO):
    """Gradients of causal attention of query rows against one KV head.

    With s_j = q.k_j/sqrt(d) over visible keys j <= pos, P = softmax(s) and
    o = sum_j P_j v_j: dv_j = P_j dO, dP_j = dO.v_j, ds_j = P_j (dP_j - dO.o),
    dq = sum_j ds_j k_j / sqrt(d), dk_j = ds_j q / sqrt(d).
    q: [n, d]; pos: [n]; K, V: [S, d]; dO: [n, d]. Returns (dq [n, d],
    dK [S, d], dV [S, d]), dK and dV summed over the rows.
    """
    q = np.asarray(q, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    n, d = q.shape
    S = K.shape[0]
    dq = np.zeros((n, d))
    dK = np.zeros((S, d))
    dV = np.zeros((S, d))
    if n == 0:
        return dq, dK, dV
    L = int(pos.max()) + 1
    s = (q @ K[:L].T) / np.sqrt(d)
    s = s + np.where(np.arange(L)[None, :] <= pos[:, None], 0.0, -np.inf)
    s = s - np.max(s, axis=1, keepdims=True)
    P = np.exp(s)
    P = P / np.sum(P, axis=1, keepdims=True)
    o = P @ V[:L]
    dV[:L] = P.T @ dO
    dP = dO @ V[:L].T
    dS = P * (dP - np.sum(dO * o, axis=1, keepdims=True))
    dq = (dS @ K[:L]) / np.sqrt(d)
    dK[:L] = (dS.T @ q) / np.sqrt(d)
    return dq, dK, dV


def prefill_bwd(Q, K, V, idx, M: int, dO_r, dO_s, positions=None):
    """Gradients of prefill (the function above) given dO_r [B, S, G, k, d]
    and dO_s [B, S, d]. A KV head's dK and dV are summed over every row that
    reads it: the selected heads of its group and, for head 0, the shared
    head ([GQA-zone] 训练与部署: shared keys/values gather the gradients of
    all their query heads). Returns (dQ [B, S, N+1, d], zero in the rows of
    unselected heads, dK [B, G, S, d], dV [B, G, S, d]).
    positions: the rows whose outputs enter the loss (default: all S). dQ
    is then returned for those rows alone ([B, P, N+1, d]) and dK, dV sum
    those rows' terms only, which is the whole gradient of every key at or
    after the first position when the positions run from there to S-1
    (earlier rows cannot see later keys).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, S, H1, d = Q.shape
    G = K.shape[1]
    k = idx.shape[-1]
    N = H1 - 1
    check_dims(N, G, k)
    pos = np.arange(S) if positions is None else np.asarray(positions, dtype=np.int64)
    rows = np.arange(pos.size)
    dQ = np.zeros((B, pos.size, H1, d))
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for g in range(G):
            for j in range(k):
                heads = g * M + idx[b, pos, g, j]
                dq, dk, dv = attend_rows_bwd(Q[b, pos, heads, :], pos, K[b, g], V[b, g], dO_r[b, pos, g, j])
                dQ[b, rows, heads, :] += dq
                dK[b, g] += dk
                dV[b, g] += dv
        dq, dk, dv = attend_rows_bwd(Q[b, pos, N, :], pos, K[b, 0], V[b, 0], dO_s[b, pos])
        dQ[b, :, N, :] += dq
        dK[b, 0] += dk
        dV[b, 0] += dv
    return dQ, dK, dV


def out_proj_bwd(O_r, w, O_s, W_O, dy, mode: str = "full"):
    """Gradients of out_proj given dy [T, D]: with A the slot vector and
    y = A W_O, dW_O = A^T dy and dA = dy W_O^T; dA splits into the hard
    slots, ō and s, and ō = sum w o feeds back into the hard slots (w dō)
    and into the routing weights (dw = o . dō), which is how the router
    receives a gradient ([GQE-review] §二: the renormalised slot).
    Ablation layouts (assemble): "hard" gives dO_r = dA and no weight
    gradient; "weighted" (A = w ⊙ O) gives dO_r = w dA and dw = o . dA, the
    gradient of the slot weights (the router probabilities p); neither reads
    the shared head, so dO_s = 0.
    Returns (dO_r [T, G, k, d], dw [T, G, k], dO_s [T, d], dW_O).
    """
    O_r = np.asarray(O_r, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, G, k, d = O_r.shape
    A = assemble(O_r, w, O_s, mode)
    dW_O = A.T @ dy
    dA = dy @ np.asarray(W_O, dtype=np.float64).T
    hard = dA[:, :G * k * d].reshape(T, G, k, d)
    if mode == "full":
        w = np.asarray(w, dtype=np.float64)
        dobar = dA[:, G * k * d:G * k * d + d]
        dO_r = hard + w[..., None] * dobar[:, None, None, :]
        dw = np.einsum("tgkd,td->tgk", O_r, dobar)
        dO_s = dA[:, G * k * d + d:]
    elif mode == "hard":
        dO_r, dw, dO_s = hard, np.zeros((T, G, k)), np.zeros((T, d))
    elif mode == "weighted":
        w = np.asarray(w, dtype=np.float64)
        dO_r = w[..., None] * hard
        dw = np.einsum("tgkd,tgkd->tgk", O_r, hard)
        dO_s = np.zeros((T, d))
    else:
        raise ValueError(f"unknown slot mode {mode!r}")
    return dO_r, dw, dO_s, dW_O


def load_balance_loss(z, idx, M: int, coef: float) -> float:
    """Auxiliary load-balancing loss of the routers ([GQE-review] §二 notes
    that training adds the standard MoE balance loss against routing
    collapse, without a formula). Reading: the usual form, per group router
    and averaged over the G groups: f_{g,m} = share of the T*k selections of
    group g that chose m, P_{g,m} = mean over tokens of p_{t,g,m};
    loss = coef * M * mean_g sum_m f_{g,m} P_{g,m}. Balanced routing with
    uniform p gives exactly coef. f is a count and carries no gradient.
    z: [T, G, M]; idx: [T, G, k].
    """
    z = np.asarray(z, dtype=np.float64)
    idx = np.asarray(idx)
    T, G, k = idx.shape
    p = softmax(z, axis=-1)
    f = np.zeros((G, M))
    for g in range(G):
        f[g] = np.bincount(idx[:, g, :].reshape(-1), minlength=M)[:M] / (T * k)
    P = p.mean(axis=0)
    return float(coef * M * np.mean(np.sum(f * P, axis=-1)))


def route_bwd(x, w_r, z, idx, dw, G: int, M: int, aux_coef: float = 0.0, wrt: str = "w"):
    """Gradients of the router given dw [T, G, k], the gradient of the slot
    weights. wrt="w": the renormalised weights of the ō slot. p = softmax(z),
    w_j = p_{m_j} / sum_{j'} p_{m_j'} over the selected experts
    ([GQE-review] §二, the w equation); the selection itself is piecewise
    constant. dp_{m_j} = (dw_j - sum_j' dw_j' w_j') / sum_j' p_{m_j'} on the
    selected experts, 0 elsewhere. wrt="p": the weights are the selected
    probabilities themselves (the weighted-concatenation ablation), so
    dp_{m_j} = dw_j. With aux_coef the balance loss (load_balance_loss) adds
    coef * M * f_{g,m} / (T * G) to dp of every expert;
    dz = p * (dp - p . dp); dW_r = dz^T x, db_r = sum_t dz, dx = dz W_r.
    x: [T, D]; w_r: [G*M, D]; z: [T, G, M]; idx: [T, G, k].
    Returns (dz [T, G, M], dW_r [G*M, D], db_r [G*M], dx [T, D]).
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    dw = np.asarray(dw, dtype=np.float64)
    T = x.shape[0]
    p = softmax(z, axis=-1)
    idx = np.asarray(idx)
    if wrt == "w":
        p_sel = np.take_along_axis(p, idx, -1)
        ssum = np.sum(p_sel, axis=-1, keepdims=True)
        wsel = p_sel / ssum
        dp_sel = (dw - np.sum(dw * wsel, axis=-1, keepdims=True)) / ssum
    elif wrt == "p":
        dp_sel = dw
    else:
        raise ValueError(f"unknown weight kind {wrt!r}")
    dp = np.zeros_like(p)
    np.put_along_axis(dp, idx, dp_sel, axis=-1)
    if aux_coef:
        k = idx.shape[-1]
        for g in range(G):
            share = np.bincount(idx[:, g, :].reshape(-1), minlength=M)[:M] / (T * k)
            dp[:, g, :] += aux_coef * M * share / (T * G)
    dz = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    dz2 = dz.reshape(T, G * M)
    w_r = np.asarray(w_r, dtype=np.float64)
    return dz, dz2.T @ x, dz2.sum(axis=0), dz2 @ w_r


def kv_bytes(B: int, L: int, G: int, d: int, S: int, b: int) -> int:
    """KV-cache bytes 2*B*L*G*S*d*b ([GQA-zone] §4.1 and §缓存省下多少).

    L is the layer count, b the bytes per element; K and V both count.
    """
    return 2 * B * L * G * S * d * b


def prefill_flops(B: int, S: int, G: int, k: int, d: int) -> int:
    """Matmul FLOP of the sparse causal prefill, counting visible pairs only.

    Per (selected row, visible key): 2d for q.k and 2d for p.v. Each token has
    G*k selected rows plus one shared row; token i sees i+1 keys.
    """
    return 4 * d * (G * k + 1) * B * S * (S + 1) // 2
