"""Plant plausible mistakes in copies of the oracle; the pins must catch each.

Each mutant is a text substitution in the oracle's source, executed as a
fresh module on the CPU. A mutant that passes every pin would mean the pins
leave that part of the oracle unfixed.
"""
import inspect
import types

import numpy as np
import pytest

import oracle.gqe_oracle as gqe_oracle
import pins

SRC = inspect.getsource(gqe_oracle)

MUTANTS = {
    "topk_ties_to_higher_index": (
        'order = np.argsort(-np.asarray(scores), axis=-1, kind="stable")',
        'order = (np.asarray(scores).shape[-1] - 1 - np.argsort(-np.asarray(scores)[..., ::-1], axis=-1, kind="stable"))'),
    "topk_smallest": (
        'order = np.argsort(-np.asarray(scores), axis=-1, kind="stable")',
        'order = np.argsort(np.asarray(scores), axis=-1, kind="stable")'),
    "topk_unsorted_slots": (
        'return np.sort(order[..., :k], axis=-1).astype(np.int64)',
        'return order[..., :k].astype(np.int64)'),
    "weights_not_renormalised": (
        "w = p_sel / np.sum(p_sel, axis=-1, keepdims=True)", "w = p_sel"),
    "weights_from_logits": (
        "p_sel = np.take_along_axis(p, idx, axis=-1)", "p_sel = np.take_along_axis(z, idx, axis=-1)"),
    "router_groups_transposed": (
        "return z.reshape(z.shape[0], G, M)", "return z.reshape(z.shape[0], M, G).transpose(0, 2, 1)"),
    "router_bias_dropped": (
        "z = z + np.asarray(b_r, dtype=np.float64)[None, :]", "z = z"),
    "scale_one_over_d": (
        "s = (qr @ K[:L].T) / np.sqrt(d)", "s = (qr @ K[:L].T) / d"),
    "mask_excludes_diagonal": (
        "np.arange(L)[None, :] <= pr[:, None]", "np.arange(L)[None, :] < pr[:, None] + (pr[:, None] == 0)"),
    "mask_one_too_many": (
        "L = int(pr.max()) + 1", "L = min(int(pr.max()) + 2, K.shape[0])\n        pr = pr + 1"),
    "head_mapping_transposed": (
        "heads = g * M + idx[b, pos, g, j]\n                O_r", "heads = idx[b, pos, g, j] * G + g\n                O_r"),
    "shared_head_on_last_group": (
        "O_s[b] = attend_rows(Qp[b, :, N, :], pos, K[b, 0], V[b, 0])",
        "O_s[b] = attend_rows(Qp[b, :, N, :], pos, K[b, G - 1], V[b, G - 1])"),
    "shared_head_uses_head0_query": (
        "O_s[b] = attend_rows(Qp[b, :, N, :], pos, K[b, 0], V[b, 0])",
        "O_s[b] = attend_rows(Qp[b, :, 0, :], pos, K[b, 0], V[b, 0])"),
    "decode_top_left_mask": (
        "pos = n - L + np.arange(L)", "pos = np.arange(L)"),
    "decode_shared_head_on_last_group": (
        "O_s[b] = attend_rows(q[b, :, N, :], pos, K[b, 0, s0:n], V[b, 0, s0:n])",
        "O_s[b] = attend_rows(q[b, :, N, :], pos, K[b, G - 1, s0:n], V[b, G - 1, s0:n])"),
    "decode_padding_ignored": (
        "        s0 = 0 if kv_start is None else int(kv_start[b])", "        s0 = 0"),
    "balance_grad_without_M": (
        "dp[:, g, :] += aux_coef * M * share / (T * G)", "dp[:, g, :] += aux_coef * share / (T * G)"),
    "balance_grad_not_averaged_over_groups": (
        "dp[:, g, :] += aux_coef * M * share / (T * G)", "dp[:, g, :] += aux_coef * M * share / T"),
    "balance_share_per_token": (
        "f[g] = np.bincount(idx[:, g, :].reshape(-1), minlength=M)[:M] / (T * k)",
        "f[g] = np.bincount(idx[:, g, :].reshape(-1), minlength=M)[:M] / T"),
    "balance_prob_summed": ("P = p.mean(axis=0)", "P = p.sum(axis=0)"),
    "lse_without_max": (
        "return top + np.log(np.sum(np.exp(sc - top[:, None]), axis=1))",
        "return np.log(np.sum(np.exp(sc - top[:, None]), axis=1))"),
    "lse_mask_excludes_diagonal": (
        "sc = np.where(np.arange(L)[None, :] <= pos[:, None], sc, -np.inf)",
        "sc = np.where(np.arange(L)[None, :] < np.maximum(pos[:, None], 1), sc, -np.inf)"),
    "lse_shared_on_last_group": (
        "lse_s[b] = lse_rows(Q[b, pos, N, :], pos, K[b, 0])", "lse_s[b] = lse_rows(Q[b, pos, N, :], pos, K[b, G - 1])"),
    "lse_head_mapping_transposed": (
        "heads = g * M + idx[b, pos, g, j]\n                lse_r", "heads = idx[b, pos, g, j] * G + g\n                lse_r"),
    "lse_positions_ignored": (
        "lse_s[b] = lse_rows(Q[b, pos, N, :], pos, K[b, 0])", "lse_s[b] = lse_rows(Q[b, pos, N, :], pos * 0 + pos.max(), K[b, 0])"),
    "bwd_head_mapping_transposed": (
        "heads = g * M + idx[b, pos, g, j]\n                dq", "heads = idx[b, pos, g, j] * G + g\n                dq"),
    "bwd_rows_take_first_gradients": (
        "V[b, g], dO_r[b, pos, g, j])", "V[b, g], dO_r[b, :pos.size, g, j])"),
    "weighted_variant_unscaled": (
        "        return (w[..., None] * O_r).reshape(T, G * k * d)",
        "        return O_r.reshape(T, G * k * d)"),
    "weighted_variant_renormalised": (
        "        return np.take_along_axis(np.asarray(p, dtype=np.float64), np.asarray(idx), axis=-1)",
        "        return np.asarray(w, dtype=np.float64)"),
    "hard_variant_keeps_shared": (
        "        return O_r.reshape(T, G * k * d)\n    if mode == \"weighted\":",
        "        return np.concatenate([O_r.reshape(T, G * k * d), np.asarray(O_s, dtype=np.float64)], axis=1)\n"
        "    if mode == \"weighted\":"),
    "weighted_variant_keeps_shared": (
        "        return (w[..., None] * O_r).reshape(T, G * k * d)",
        "        return np.concatenate([(w[..., None] * O_r).reshape(T, G * k * d), np.asarray(O_s, dtype=np.float64)], axis=1)"),
    "ablation_rows_keep_shared": (
        "    if mode in (\"hard\", \"weighted\"):\n        return G * k * d",
        "    if mode in (\"hard\", \"weighted\"):\n        return (G * k + 1) * d"),
    "ablation_bwd_shared_gradient": (
        "        dO_r, dw, dO_s = hard, np.zeros((T, G, k)), np.zeros((T, d))",
        "        dO_r, dw, dO_s = hard, np.zeros((T, G, k)), np.ones((T, d))"),
    "route_bwd_p_renormalised": (
        "    elif wrt == \"p\":\n        dp_sel = dw",
        "    elif wrt == \"p\":\n        p_sel = np.take_along_axis(p, idx, -1)\n"
        "        dp_sel = (dw - np.sum(dw * p_sel / p_sel.sum(-1, keepdims=True), axis=-1, keepdims=True)) / p_sel.sum(-1, keepdims=True)"),
    "bwd_softmax_without_delta": (
        "    dS = P * (dP - np.sum(dO * o, axis=1, keepdims=True))", "    dS = P * dP"),
    "bwd_key_scale_missing": (
        "    dK[:L] = (dS.T @ q) / np.sqrt(d)", "    dK[:L] = dS.T @ q"),
    "bwd_shared_head_on_last_group": (
        "        dK[b, 0] += dk\n", "        dK[b, G - 1] += dk\n"),
    "bwd_obar_not_fed_back": (
        "        dO_r = hard + w[..., None] * dobar[:, None, None, :]", "        dO_r = hard"),
    "bwd_router_not_renormalised": (
        "    dp_sel = (dw - np.sum(dw * wsel, axis=-1, keepdims=True)) / ssum", "    dp_sel = dw / ssum"),
    "obar_mean_over_groups": (
        "        obar = np.sum(w[..., None] * O_r, axis=(1, 2))",
        "        obar = np.sum(w[..., None] * O_r, axis=(1, 2)) / G"),
    "obar_group0_only": (
        "        obar = np.sum(w[..., None] * O_r, axis=(1, 2))",
        "        obar = np.sum(w[:, 0, :, None] * O_r[:, 0], axis=1)"),
    "obar_unweighted": (
        "        obar = np.sum(w[..., None] * O_r, axis=(1, 2))",
        "        obar = np.sum(O_r, axis=(1, 2))"),
    "hard_slots_slot_major": (
        "hard = O_r.reshape(T, G * k * d)", "hard = O_r.transpose(0, 2, 1, 3).reshape(T, G * k * d)"),
    "slot_parts_swapped": (
        "return np.concatenate([hard, obar, shared], axis=1)",
        "return np.concatenate([hard, shared, obar], axis=1)"),
    "kv_bytes_without_factor_2": (
        "return 2 * B * L * G * S * d * b", "return B * L * G * S * d * b"),
    "lists_descending": (
        "tok[b, g, pos:pos + rows.size] = rows", "tok[b, g, pos:pos + rows.size] = rows[::-1]"),
    "reject_nothing": (
        "if G <= 0 or N <= 0 or N % G != 0:", "if G <= 0 or N <= 0:"),
    "proj_head_mapping_transposed": (
        "        g, m = divmod(h, M)", "        m, g = divmod(h, G)"),
    "proj_shared_head_from_block0": (
        "    Q[:, :, N] = x @ Wq[N].T", "    Q[:, :, N] = x @ Wq[0].T"),
    "proj_every_head_computed": (
        "        Q[chose, h] = x[chose] @ Wq[h].T", "        Q[:, :, h] = x @ Wq[h].T"),
    "proj_k_layout_token_major": (
        "K = (x @ np.asarray(W_K, dtype=np.float64).T).reshape(B, S, G, d).transpose(0, 2, 1, 3)",
        "K = (x @ np.asarray(W_K, dtype=np.float64).T).reshape(B, G, S, d)"),
    "proj_v_from_key_weights": (
        "V = (x @ np.asarray(W_V, dtype=np.float64).T)", "V = (x @ np.asarray(W_K, dtype=np.float64).T)"),
    "decode_append_at_cache_start": (
        "        Kc[b, :, n - L:n] = K[b]", "        Kc[b, :, 0:L] = K[b]"),
    "proj_flops_without_shared_head": (
        "return 2 * T * D * ((G * k + 1) * d + 2 * G * d)", "return 2 * T * D * (G * k * d + 2 * G * d)"),
    "flops_strict_triangle": (
        "return 4 * d * (G * k + 1) * B * S * (S + 1) // 2", "return 4 * d * (G * k + 1) * B * S * (S - 1) // 2"),
}


def _mutant_module(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutant {name}: anchor must occur exactly once"
    mod = types.ModuleType(f"gqe_oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant_module(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches the planted mistake '{name}'"
