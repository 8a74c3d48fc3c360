"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Tolerances: bf16 inputs with fp32 accumulation -> max |error| <= 2e-2 and
relative Frobenius error <= 1e-2; fp32 -> max |error| <= 1e-5. Routing
indices and token lists are compared bit for bit. Small cases are compared
element by element; the full-size workloads (run in the launch configuration
the benchmark times) are compared on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_query_gqa_amd as gqe
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
f64 = synth.to_f64


def tol(dtype):
    return (2e-2, 1e-2) if dtype == "bf16" else (1e-5, 1e-6)


def assert_close(got, ref, dtype, what):
    got = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    amax, rel = tol(dtype)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)) if got.size else 0.0
    print(f"{what}: max|err|={err:.3e} rel_fro={fro:.3e}")
    assert err <= amax, f"{what}: max abs error {err:.3e} > {amax}"
    assert fro <= rel, f"{what}: relative Frobenius error {fro:.3e} > {rel}"


def to_dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def dims_of(cfg, **kw):
    c = cfg.replace(**kw) if kw else cfg
    return gqe.gqe_dims.from_config(c)


def small_cfg(B, S, D, N, G, k, d, dtype="bf16", seed=0, skew=False):
    return synth.GQEConfig("case", B=B, S=S, D=D, N=N, G=G, k=k, d=d, dtype=dtype, seed=seed, skew=skew)


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,S,D,G,M,k", [(1, 1, 8, 1, 1, 1), (2, 77, 40, 3, 4, 2), (1, 130, 64, 8, 2, 1),
                                         (3, 64, 96, 2, 32, 5), (1, 200, 256, 8, 32, 32),
                                         (2, 150, 128, 16, 16, 3),
                                         # at most 16 tokens (one token tile per block) and just past
                                         (2, 8, 512, 8, 4, 2), (4, 4, 4096, 8, 32, 3), (16, 1, 1024, 16, 8, 2),
                                         (1, 17, 96, 2, 8, 2)])
def test_route_exact_with_ties(dtype, B, S, D, G, M, k):
    """Integer-valued x and W_r make every logit exact in fp32, so the
    selection must equal the oracle's bit for bit, planted ties included
    (duplicate expert rows; all-zero tokens whose logits all tie)."""
    rng = np.random.default_rng(B * 1000 + S)
    T = B * S
    x = rng.integers(-3, 4, size=(T, D)).astype(np.float32)
    x[::7] = 0.0
    w = rng.integers(-2, 3, size=(G * M, D)).astype(np.float32)
    if M > 1:
        w[1::M] = w[0::M]  # expert 1 duplicates expert 0 in every group
    bias = (rng.integers(-4, 5, size=G * M) * 0.5).astype(np.float32)
    if M > 2:
        bias[2::M] = bias[0::M]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xt, wt = torch.from_numpy(x).to(tdt), torch.from_numpy(w).to(tdt)
    dims = gqe.gqe_dims.make(B, S, D, G * M, G, k, 32, dtype)
    out = gqe.route(dims, xt.to(DEV), wt.to(DEV), torch.from_numpy(bias).to(DEV), want_p=True)
    torch.cuda.synchronize()
    z = oracle.route_logits(x, w, G, M, bias)
    p, idx, wref = oracle.route_select(z, k)
    assert np.array_equal(out["logits"].cpu().numpy().astype(np.float64), z), "logits not exact"
    assert np.array_equal(out["topk_idx"].cpu().numpy(), idx), "selection differs"
    assert np.max(np.abs(f64(out["topk_w"]) - wref)) <= 1e-6
    assert np.max(np.abs(f64(out["topk_p"]) - oracle.slot_weights(p, idx, wref, "weighted"))) <= 1e-6
    if k == 1:
        assert torch.all(out["topk_w"] == 1.0)
    off, tok = oracle.build_lists(idx.reshape(B, S, G, k), M)
    assert np.array_equal(out["list_off"].cpu().numpy(), off)
    assert np.array_equal(out["list_tok"].cpu().numpy(), tok)


def _route_check(cfg, inp, out):
    """Logits within the fp32 bound; indices equal the oracle's wherever the
    fp64 top-k margin exceeds twice that bound; lists equal the oracle's
    lists on every (b, g) without an excluded near-tie; and the GPU's
    selection is consistent with its own logits."""
    T, G, M, k = cfg.T, cfg.G, cfg.M, cfg.k
    x, w = f64(inp["x"]), f64(inp["w_r"])
    b = None if inp["b_r"] is None else f64(inp["b_r"])
    z = oracle.route_logits(x, w, G, M, b)
    p, idx, wref = oracle.route_select(z, k)
    zg = f64(out["logits"])
    scale = (np.abs(x) @ np.abs(w).T).reshape(T, G, M) + 1.0
    bound = 1e-5 * scale
    assert np.all(np.abs(zg - z) <= bound), f"logit error {np.max(np.abs(zg - z) / scale):.3e}"
    gidx = out["topk_idx"].cpu().numpy()
    # A (token, group) can only select differently if its fp64 top-k margin is
    # at most twice the largest logit error in that row; every other pair
    # must match bit for bit.
    srt = np.sort(z, -1)
    margin = (srt[..., M - k] - srt[..., M - k - 1]) if k < M else np.full((T, G), np.inf)
    row_err = np.abs(zg - z).max(-1)
    ok = margin > 2 * row_err
    n_excl = int((~ok).sum())
    n_diff = int(np.any(gidx != idx, axis=-1).sum())
    print(f"{cfg.name}: max logit err/scale {np.max(np.abs(zg - z) / scale):.2e}; "
          f"{n_excl} near-tie (token, group) pairs of {T * G} excluded; {n_diff} differ in total")
    assert np.array_equal(gidx[ok], idx[ok]), "selection differs outside near-ties"
    assert n_excl <= max(2, 1e-4 * T * G)
    assert np.max(np.abs(f64(out["topk_w"])[ok] - wref[ok])) <= 2e-5
    if out.get("topk_p") is not None:
        pref = oracle.slot_weights(p, idx, wref, "weighted")
        assert np.max(np.abs(f64(out["topk_p"])[ok] - pref[ok])) <= 2e-5
    # GPU selection vs GPU logits: selected >= unselected, ties to lower index
    sel = np.zeros((T, G, M), bool)
    np.put_along_axis(sel, gidx.astype(np.int64), True, -1)
    assert np.all(np.diff(gidx, axis=-1) > 0)
    if k < M:
        lo = np.where(sel, zg, np.inf).min(-1)
        hi = np.where(sel, -np.inf, zg).max(-1)
        assert np.all(lo >= hi)
    if cfg.mode == "prefill":
        S = cfg.S
        off, tok = oracle.build_lists(gidx.reshape(cfg.B, S, G, k), M)
        assert np.array_equal(out["list_off"].cpu().numpy(), off)
        assert np.array_equal(out["list_tok"].cpu().numpy(), tok)
        off_o, _ = oracle.build_lists(idx.reshape(cfg.B, S, G, k), M)
        okbg = ok.reshape(cfg.B, S, G).all(1)
        assert np.array_equal(out["list_off"].cpu().numpy()[okbg], off_o[okbg])
        counts = np.diff(out["list_off"].cpu().numpy(), axis=-1)
        print(f"{cfg.name}: per-(g, m) token counts, sequence 0: {counts[0].tolist()}")


@pytest.mark.parametrize("name", ["tiny_f32", "main_s2k", "long_s128k", "llama_s8k_skew", "decode_kv64k"])
def test_route_workloads(name):
    cfg = synth.workload(name)
    if cfg.mode == "decode":
        rng = np.random.default_rng(cfg.seed)
        x = synth.round_bf16(rng.standard_normal((cfg.T, cfg.D), dtype=np.float32))
        rng.standard_normal(((cfg.N + 1) * cfg.d, cfg.D), dtype=np.float32)  # W_Q draw
        w_r = synth.round_bf16(rng.standard_normal((cfg.G * cfg.M, cfg.D), dtype=np.float32) * np.float32(0.02))
        inp = dict(x=x, w_r=w_r, b_r=None)
        dims = gqe.gqe_dims.make(cfg.B, cfg.q_len, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.dtype)
        out = gqe.route(dims, x.to(DEV), w_r.to(DEV), None, want_lists=False, want_p=True)
    else:
        inp = synth.make_prefill_inputs(cfg)
        out = gqe.route(dims_of(cfg), inp["x"].to(DEV), inp["w_r"].to(DEV),
                        None if inp["b_r"] is None else inp["b_r"].to(DEV), want_p=True)
    torch.cuda.synchronize()
    _route_check(cfg, inp, out)


# ---------------------------------------------------------------------------
# Prefill attention
# ---------------------------------------------------------------------------

PREFILL_CASES = [
    # B, S, D, N, G, k, d, dtype, peaked
    (1, 1, 64, 4, 2, 1, 32, "f32", False),
    (1, 128, 256, 4, 2, 1, 32, "f32", False),
    (2, 77, 64, 8, 2, 3, 64, "f32", True),
    (1, 150, 64, 6, 6, 1, 128, "f32", False),
    (1, 1, 64, 4, 2, 1, 64, "bf16", False),
    (1, 7, 64, 8, 1, 2, 64, "bf16", False),
    (2, 300, 128, 16, 8, 1, 64, "bf16", False),
    (2, 300, 128, 16, 8, 1, 64, "bf16", True),
    (1, 517, 128, 32, 8, 2, 128, "bf16", False),
    (1, 517, 128, 32, 8, 2, 128, "bf16", True),
    (3, 200, 64, 8, 4, 2, 32, "bf16", True),
    (1, 129, 64, 8, 8, 1, 64, "bf16", False),
    (1, 64, 64, 16, 4, 4, 64, "bf16", False),
    # MHA (M = 1) and dense MQA (G = 1, k = M) at d = 128
    (2, 100, 64, 8, 8, 1, 128, "bf16", False),
    (1, 300, 64, 4, 1, 4, 128, "bf16", True),
]


def _prefill_inputs(cfg, peaked):
    inp = synth.make_prefill_inputs(cfg)
    if peaked:  # sharpen the softmax: power-of-two scaling is exact in bf16
        inp["q"] = inp["q"] * 8
    # distinct KV heads: offset V of group g by 0.25*g, which keeps |o| small enough
    # that output rounding stays far below the absolute bounds
    off = (0.25 * torch.arange(cfg.G, dtype=torch.float32)).view(1, cfg.G, 1, 1)
    inp["v"] = (inp["v"].float() + off).to(cfg.torch_dtype)
    inp["idx"] = synth.random_selection(cfg.B, cfg.S, cfg.G, cfg.M, cfg.k, cfg.seed + 5)
    return inp


# The bf16 d <= 64 kernel has two forms (plain, and key-split for launches
# with few tiles); the launcher picks by tile count unless GQE_PREFILL_FORM
# forces one. Cases of that kernel run under each form.
FORMS = ["auto", "plain", "split"]


def _with_forms(cases, d_of, dtype_of=lambda c: "bf16"):
    """(case, form) pairs: every case under the launcher's own choice, and the
    bf16 d <= 64 cases also under each forced form (the d = 128 and fp32
    kernels have one form)."""
    return [pytest.param(c, f, id="-".join(map(str, c)) + "-" + f)
            for c in cases for f in FORMS if f == "auto" or (d_of(c) <= 64 and dtype_of(c) == "bf16")]


def _set_form(monkeypatch, form, d, dtype):
    assert form == "auto" or (d <= 64 and dtype == "bf16")
    if form == "auto":
        monkeypatch.delenv("GQE_PREFILL_FORM", raising=False)
    else:
        monkeypatch.setenv("GQE_PREFILL_FORM", form)


@pytest.mark.parametrize("case,form", _with_forms(PREFILL_CASES, lambda c: c[6], lambda c: c[7]))
def test_prefill_small(case, form, monkeypatch):
    B, S, D, N, G, k, d, dtype, peaked = case
    _set_form(monkeypatch, form, d, dtype)
    cfg = small_cfg(B, S, D, N, G, k, d, dtype)
    inp = _prefill_inputs(cfg, peaked)
    g = to_dev(inp)
    o_r, o_s = gqe.prefill(dims_of(cfg), g["q"], g["k"], g["v"], g["idx"])
    torch.cuda.synchronize()
    idx = inp["idx"].numpy().reshape(B, S, G, k)
    ref_r, ref_s = oracle.prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), idx, cfg.M)
    assert_close(o_r, ref_r, dtype, "O_routed")
    assert_close(o_s, ref_s, dtype, "O_shared")


# Scores that rise (or fall) steeply along the sequence: the kernels' reference
# max must move many times after the first key block (rising), or stay far
# above most later scores (falling). Keys are a ramp a_j along one direction u
# plus noise; every query is u plus noise, so the log2-domain scores
# log2(e) * q.k / sqrt(d) span about 1500 over the sequence.
RAMP_CASES = [
    # B, S, D, N, G, k, d, rising
    (3, 200, 64, 8, 4, 2, 32, True),
    (2, 300, 128, 16, 8, 1, 64, True),
    (2, 300, 128, 16, 8, 1, 64, False),
    (1, 517, 128, 32, 8, 2, 128, True),
    (1, 517, 128, 32, 8, 2, 128, False),
]


@pytest.mark.parametrize("case,form", _with_forms(RAMP_CASES, lambda c: c[6]))
def test_prefill_reference_moves(case, form, monkeypatch):
    B, S, D, N, G, k, d, rising = case
    _set_form(monkeypatch, form, d, "bf16")
    cfg = small_cfg(B, S, D, N, G, k, d)
    inp = _prefill_inputs(cfg, False)
    gen = torch.Generator().manual_seed(11)
    u = torch.ones(d)
    q = u + 0.1 * torch.randn(B, S, N + 1, d, generator=gen)
    j = torch.arange(S, dtype=torch.float32)
    a = 1500.0 * (j if rising else (S - 1 - j)) / (S * 1.4426950408889634 * d ** 0.5)
    kk = a.view(1, 1, S, 1) * u + 0.5 * torch.randn(B, G, S, d, generator=gen)
    inp["q"], inp["k"] = q.to(cfg.torch_dtype), kk.to(cfg.torch_dtype)
    g = to_dev(inp)
    o_r, o_s = gqe.prefill(dims_of(cfg), g["q"], g["k"], g["v"], g["idx"])
    torch.cuda.synchronize()
    idx = inp["idx"].numpy().reshape(B, S, G, k)
    ref_r, ref_s = oracle.prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), idx, cfg.M)
    assert_close(o_r, ref_r, "bf16", "O_routed")
    assert_close(o_s, ref_s, "bf16", "O_shared")


def _sample_positions(S, n=256, seed=1):
    if S <= n:
        return np.arange(S)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, S - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, S - 1], mid]))


@pytest.mark.parametrize("name", ["main_s2k", "long_s128k", "llama_s8k_skew"])
def test_prefill_workloads_sampled(name):
    """Every sequence of each workload, in the launch configuration the
    benchmark times. 2048-token sequences (8 of them, each with its shared
    tiles on its own XCD list) are compared on every row; longer ones on 256
    sampled positions (first and last included)."""
    cfg = synth.workload(name)
    inp = synth.make_prefill_inputs(cfg)
    inp["idx"] = synth.random_selection(cfg.B, cfg.S, cfg.G, cfg.M, cfg.k, cfg.seed, skew=cfg.skew)
    g = to_dev(inp)
    o_r, o_s = gqe.prefill(dims_of(cfg), g["q"], g["k"], g["v"], g["idx"])
    torch.cuda.synchronize()
    full = cfg.S <= 2048
    pos = np.arange(cfg.S) if full else _sample_positions(cfg.S)
    idx = inp["idx"].numpy().reshape(cfg.B, cfg.S, cfg.G, cfg.k)
    what = "every row" if full else "sampled"
    for b in range(cfg.B):
        ref_r, ref_s = oracle.prefill(f64(inp["q"][b:b + 1]), f64(inp["k"][b:b + 1]), f64(inp["v"][b:b + 1]),
                                      idx[b:b + 1], cfg.M, positions=None if full else pos)
        assert_close(o_r[b:b + 1, pos], ref_r, cfg.dtype, f"{name} b={b} O_routed ({what})")
        assert_close(o_s[b:b + 1, pos], ref_s, cfg.dtype, f"{name} b={b} O_shared ({what})")


def test_prefill_million_tokens_sampled():
    """One sequence of 1,048,576 tokens (the far end of the pages' 4k-1024k
    range; the long-context layer's shape), in the launch configuration the
    benchmark times: q, k and v drawn directly (too long to project on the
    host), rows at tile edges, powers of two, the middle and the end, and a
    few random positions against the oracle's full causal sums."""
    cfg = synth.workload("long_s1m")
    S = cfg.S
    inp = synth.make_attention_inputs(cfg)
    idx = synth.random_selection(cfg.B, S, cfg.G, cfg.M, cfg.k, 13)
    print("long_s1m: inputs made", flush=True)
    q, kk, vv = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    o_r, o_s = gqe.prefill(dims_of(cfg), q, kk, vv, idx.to(DEV))
    torch.cuda.synchronize()
    print("long_s1m: kernel done", flush=True)
    rng = np.random.default_rng(17)
    pos = np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, 65535, 65536, S // 2 - 1, S // 2, S - 2, S - 1],
                                    rng.choice(np.arange(S), size=4, replace=False)]))
    ref_r, ref_s = oracle.prefill(f64(inp["q"][:, torch.from_numpy(pos)]), f64(inp["k"]), f64(inp["v"]),
                                  idx.numpy().reshape(1, S, cfg.G, cfg.k), cfg.M, positions=pos, q_rows_only=True)
    assert_close(o_r[:, pos], ref_r, cfg.dtype, f"long_s1m O_routed ({pos.size} positions)")
    assert_close(o_s[:, pos], ref_s, cfg.dtype, f"long_s1m O_shared ({pos.size} positions)")


# Sequences past 8k tokens with ragged row counts: tile edges, skewed lists
# and the striped tile order (G not a multiple of 8).
LONG_FORM_CASES = [
    # B, S, D, N, G, k, d, skew
    (2, 8269, 64, 16, 8, 2, 64, True),   # ragged rows, two slots per token, skewed lists
    (1, 8192, 64, 4, 2, 1, 64, False),   # G not a multiple of 8: striped tile order
    (1, 9000, 64, 8, 8, 1, 64, False),   # one expert per group (k = M)
    (1, 16384, 64, 16, 8, 1, 32, False),  # d = 32 with 576 tiles: the plain form when not forced
]


@pytest.mark.parametrize("case,form", _with_forms(LONG_FORM_CASES, lambda c: c[6]))
def test_prefill_long_form(case, form, monkeypatch):
    """Rows around every 256-row tile edge, the first and last rows and a
    random sample, against the oracle; also the training forward's lse."""
    B, S, D, N, G, k, d, skew = case
    _set_form(monkeypatch, form, d, "bf16")
    cfg = small_cfg(B, S, D, N, G, k, d, seed=7, skew=skew)
    inp = _prefill_inputs(cfg, peaked=False)
    inp["idx"] = synth.random_selection(B, S, G, cfg.M, k, 11, skew=skew)
    g = to_dev(inp)
    dims = dims_of(cfg)
    o_r, o_s = gqe.prefill(dims, g["q"], g["k"], g["v"], g["idx"])
    t_r, t_s, lse_r, lse_s = gqe.prefill_train(dims, g["q"], g["k"], g["v"], g["idx"])
    torch.cuda.synchronize()
    assert torch.equal(o_r, t_r) and torch.equal(o_s, t_s)
    # token positions at the edges of 256-row tiles (routed rows are k per token)
    edges = set()
    for rows in (S * k, S):
        per = k if rows == S * k else 1
        for e in range(0, rows, 256):
            for r in (e - 1, e, e + 1):
                if 0 <= r < rows:
                    edges.add(r // per)
    rng = np.random.default_rng(S)
    extra = rng.choice(np.arange(S), size=64, replace=False)
    pos = np.unique(np.concatenate([sorted(edges), extra, np.arange(S - 40, S), np.arange(40)]))
    idx = inp["idx"].numpy().reshape(B, S, G, k)
    print(f"case {case}: {pos.size} positions", flush=True)
    for b in range(B):
        Q, K, V = f64(inp["q"][b:b + 1]), f64(inp["k"][b:b + 1]), f64(inp["v"][b:b + 1])
        ref_r, ref_s = oracle.prefill(Q, K, V, idx[b:b + 1], cfg.M, positions=pos)
        assert_close(o_r[b:b + 1, pos], ref_r, cfg.dtype, f"b={b} O_routed")
        assert_close(o_s[b:b + 1, pos], ref_s, cfg.dtype, f"b={b} O_shared")
        lr, ls = oracle.prefill_lse(Q, K, idx[b:b + 1], cfg.M, positions=pos)
        for got, ref, name in ((lse_r[b:b + 1, pos], lr, "lse_r"), (lse_s[b:b + 1, pos], ls, "lse_s")):
            e = np.abs(f64(got) - ref) / np.maximum(1.0, np.abs(ref))
            print(f"b={b} {name}: max scaled err {float(e.max()):.3e}")
            assert float(e.max()) <= 2e-2, name


def test_prefill_deterministic():
    cfg = small_cfg(2, 300, 128, 16, 8, 1, 64)
    inp = to_dev(_prefill_inputs(cfg, False))
    a = gqe.prefill(dims_of(cfg), inp["q"], inp["k"], inp["v"], inp["idx"])
    b = gqe.prefill(dims_of(cfg), inp["q"], inp["k"], inp["v"], inp["idx"])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_prefill_causal_and_compaction():
    """Token i's outputs ignore later tokens and other tokens' routing."""
    cfg = small_cfg(1, 260, 64, 8, 2, 2, 64)
    inp = _prefill_inputs(cfg, False)
    g = to_dev(inp)
    a_r, a_s = gqe.prefill(dims_of(cfg), g["q"], g["k"], g["v"], g["idx"])
    i = 131
    q2, k2, v2 = g["q"].clone(), g["k"].clone(), g["v"].clone()
    q2[:, i + 1:] = -q2[:, i + 1:]
    k2[:, :, i + 1:] = k2[:, :, i + 1:] * 2
    v2[:, :, i + 1:] = v2[:, :, i + 1:] + 1
    idx2 = synth.random_selection(1, 260, 2, 4, 2, 99).to(DEV)
    idx2[i] = g["idx"][i]
    b_r, b_s = gqe.prefill(dims_of(cfg), q2, k2, v2, idx2)
    assert torch.equal(a_r[:, i], b_r[:, i]) and torch.equal(a_s[:, i], b_s[:, i])


# ---------------------------------------------------------------------------
# Decode attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 8])
@pytest.mark.parametrize("q_len", [1, 2])
def test_decode_boundary_matrix(dtype, G, q_len):
    """q_len in {1, 2}, kv_len in {7, 17} (plus one long ragged length),
    G in {1, 2, H} with H = 8, distinct KV heads."""
    H, d, Smax = 8, 64, 300
    M = H // G
    k = min(M, 2 if q_len == 1 else 1)
    B = 3
    rng = np.random.default_rng(G * 10 + q_len)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, q_len, H + 1, d), dtype=np.float32)).to(tdt)
    kc = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    vc = torch.from_numpy((rng.standard_normal((B, G, Smax, d)) + 0.25 * np.arange(G)[None, :, None, None]).astype(np.float32)).to(tdt)
    kv_len = np.array([7, 17, 293], dtype=np.int32)
    idx = synth.random_selection(B, q_len, G, M, k, 3)
    dims = gqe.gqe_dims.make(B, Smax, 64, H, G, k, d, dtype)
    o_r, o_s = gqe.decode(dims, q_len, q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(kv_len).to(DEV),
                          idx.to(DEV))
    torch.cuda.synchronize()
    ref_r, ref_s = oracle.decode(f64(q), f64(kc), f64(vc), kv_len, idx.numpy().reshape(B, q_len, G, k), M)
    assert_close(o_r, ref_r, dtype, f"decode G={G} q_len={q_len} O_routed")
    assert_close(o_s, ref_s, dtype, f"decode G={G} q_len={q_len} O_shared")


# Decode with many query rows per (sequence, group): (k+1)*q_len up to the
# 16-row limit, which selects the 8- and 16-row kernel instantiations.
@pytest.mark.parametrize("dtype,d,H,G,k,q_len", [("bf16", 64, 16, 2, 3, 2), ("bf16", 128, 16, 2, 7, 2),
                                                 ("bf16", 32, 8, 2, 3, 4), ("f32", 64, 16, 2, 7, 2),
                                                 ("f32", 128, 8, 1, 3, 3), ("bf16", 128, 32, 4, 5, 2)])
def test_decode_many_rows(dtype, d, H, G, k, q_len):
    M = H // G
    B, Smax = 2, 700
    rng = np.random.default_rng(d + 7 * k + q_len)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, q_len, H + 1, d), dtype=np.float32)).to(tdt)
    kc = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    vc = torch.from_numpy((rng.standard_normal((B, G, Smax, d)) + 0.25 * np.arange(G)[None, :, None, None]).astype(np.float32)).to(tdt)
    kv_len = np.array([q_len + 3, 651], dtype=np.int32)
    idx = synth.random_selection(B, q_len, G, M, k, 9)
    dims = gqe.gqe_dims.make(B, Smax, 64, H, G, k, d, dtype)
    o_r, o_s = gqe.decode(dims, q_len, q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(kv_len).to(DEV),
                          idx.to(DEV))
    torch.cuda.synchronize()
    ref_r, ref_s = oracle.decode(f64(q), f64(kc), f64(vc), kv_len, idx.numpy().reshape(B, q_len, G, k), M)
    assert_close(o_r, ref_r, dtype, f"decode rows={(k + 1) * q_len} d={d} O_routed")
    assert_close(o_s, ref_s, dtype, f"decode rows={(k + 1) * q_len} d={d} O_shared")


def test_decode_matches_prefill_rows():
    """Decode of the token at position p against p+1 cached keys equals row p
    of the prefill (a property that holds at any size)."""
    cfg = small_cfg(2, 333, 64, 16, 8, 1, 64)
    inp = to_dev(_prefill_inputs(cfg, False))
    o_r, o_s = gqe.prefill(dims_of(cfg), inp["q"], inp["k"], inp["v"], inp["idx"])
    for p in (0, 63, 64, 200, 332):
        idx_p = inp["idx"].view(2, 333, 8, 1)[:, p].contiguous().view(2, 8, 1)
        kv_len = torch.full((2,), p + 1, dtype=torch.int32, device=DEV)
        d_r, d_s = gqe.decode(dims_of(cfg), 1, inp["q"][:, p:p + 1].contiguous(), inp["k"], inp["v"],
                              kv_len, idx_p)
        assert_close(d_r[:, 0], f64(o_r[:, p]), "bf16", f"decode vs prefill p={p}")
        assert_close(d_s[:, 0], f64(o_s[:, p]), "bf16", f"decode vs prefill shared p={p}")


def test_decode_workload():
    """All 16 sequences of the 64k-key decode, every output, in the launch
    configuration the benchmark times."""
    cfg = synth.workload("decode_kv64k")
    inp = synth.make_decode_inputs(cfg)
    idx = synth.random_selection(cfg.B, cfg.q_len, cfg.G, cfg.M, cfg.k, cfg.seed)
    g = to_dev(inp)
    o_r, o_s = gqe.decode(dims_of(cfg), cfg.q_len, g["q"], g["k"], g["v"], g["kv_len"], idx.to(DEV))
    torch.cuda.synchronize()
    idx4 = idx.numpy().reshape(cfg.B, cfg.q_len, cfg.G, cfg.k)
    for b in range(cfg.B):
        ref_r, ref_s = oracle.decode(f64(inp["q"][b:b + 1]), f64(inp["k"][b:b + 1]), f64(inp["v"][b:b + 1]),
                                     inp["kv_len"].numpy()[b:b + 1], idx4[b:b + 1], cfg.M)
        assert_close(o_r[b:b + 1], ref_r, cfg.dtype, f"decode b={b} O_routed")
        assert_close(o_s[b:b + 1], ref_s, cfg.dtype, f"decode b={b} O_shared")


@pytest.mark.parametrize("d,q_len", [(128, 1), (64, 2), (32, 1)])
def test_decode_deterministic(d, q_len):
    """Two decode calls on the same inputs give the same bits: the split
    partials are merged in a fixed order with no atomics. The second call
    gets a workspace filled with NaN, so a combine that read a partial its
    own split pass did not write would show."""
    B, Smax, H, G, k = 4, 40000, 16, 8, 2
    rng = np.random.default_rng(d + q_len)
    bf = torch.bfloat16
    q = torch.from_numpy(rng.standard_normal((B, q_len, H + 1, d), dtype=np.float32)).to(bf).to(DEV)
    K = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(bf).to(DEV)
    V = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(bf).to(DEV)
    kv_len = torch.tensor([40000, 4097, 2, 23456], dtype=torch.int32, device=DEV)
    idx = synth.random_selection(B, q_len, G, H // G, k, 5).to(DEV)
    dims = gqe.gqe_dims.make(B, Smax, 64, H, G, k, d, "bf16")
    a_r, a_s = gqe.decode(dims, q_len, q, K, V, kv_len, idx)
    ws = gqe.decode_workspace(dims, q_len, DEV)
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    b_r, b_s = gqe.decode(dims, q_len, q, K, V, kv_len, idx, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a_r, b_r) and torch.equal(a_s, b_s)
    assert bool(torch.isfinite(a_r.float()).all()) and bool(torch.isfinite(a_s.float()).all())


# ---------------------------------------------------------------------------
# Slot assembly + W_O
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,G,k,d,D,dtype", [(1, 2, 1, 32, 256, "f32"), (130, 2, 2, 64, 72, "f32"),
                                             (1, 8, 1, 64, 1024, "bf16"), (300, 8, 1, 64, 1024, "bf16"),
                                             (257, 8, 2, 128, 136, "bf16"), (64, 1, 1, 32, 8, "bf16"),
                                             (129, 4, 3, 32, 264, "bf16"),
                                             # few-token kernel: ragged column tiles, several DMA passes
                                             (16, 8, 2, 128, 4096, "bf16"), (7, 2, 3, 32, 72, "bf16"),
                                             (16, 1, 1, 32, 8, "bf16"), (5, 4, 2, 64, 136, "bf16"),
                                             (11, 32, 4, 128, 264, "bf16"),
                                             # GEMM kernel: d=32, ragged columns and tokens
                                             (256, 2, 3, 32, 264, "bf16"), (1000, 4, 2, 128, 8, "bf16"),
                                             # 64-k GEMM form (d=64): 16 and 9 hard slots, ragged tiles
                                             (513, 8, 2, 64, 264, "bf16"), (700, 3, 3, 64, 520, "bf16"),
                                             # obar from registers: its steps among the first stages
                                             # (d=64, one slot), right after them (two slots at d=64,
                                             # one at d=128)
                                             (600, 1, 1, 64, 520, "bf16"), (256, 2, 1, 64, 264, "bf16"),
                                             (300, 1, 1, 128, 264, "bf16")])
def test_out_proj_small(T, G, k, d, D, dtype):
    s = synth.make_slot_inputs(T, G, k, d, D, dtype, seed=T)
    g = to_dev(s)
    dims = gqe.gqe_dims.make(1, T, D, G * k, G, k, d, dtype)
    y = gqe.out_proj(dims, T, g["o_r"], g["w"], g["o_s"], g["w_o"])
    torch.cuda.synchronize()
    ref = oracle.out_proj(f64(s["o_r"]), f64(s["w"]), f64(s["o_s"]), f64(s["w_o"]))
    assert_close(y, ref, dtype, f"out_proj T={T}")


# Token tiles whose workgroup takes several 256-column tiles (obar formed once
# for them): the group size is chosen from the tile count, and on a 256-CU
# device these sizes give four column tiles per workgroup (d = 64, ragged last
# column tile and token tile), eight (d = 128) and four (one slot at d = 64,
# where every column tile's first stages hold the obar steps).
@pytest.mark.parametrize("T,G,k,d,D", [(65613, 8, 1, 64, 1000), (66000, 8, 2, 128, 2048),
                                       (70000, 1, 1, 64, 1024)])
def test_out_proj_column_groups(T, G, k, d, D):
    s = synth.make_slot_inputs(T, G, k, d, D, "bf16", seed=T)
    g = to_dev(s)
    dims = gqe.gqe_dims.make(1, T, D, G * k, G, k, d, "bf16")
    y = gqe.out_proj(dims, T, g["o_r"], g["w"], g["o_s"], g["w_o"])
    torch.cuda.synchronize()
    ref = oracle.out_proj(f64(s["o_r"]), f64(s["w"]), f64(s["o_s"]), f64(s["w_o"]))
    assert_close(y, ref, "bf16", f"out_proj T={T} D={D} (column groups)")


@pytest.mark.parametrize("mode", ["hard", "weighted"])
@pytest.mark.parametrize("T,G,k,d,D,dtype", [(5, 4, 2, 64, 136, "bf16"), (16, 8, 2, 128, 4096, "bf16"),
                                             (100, 8, 2, 64, 264, "bf16"), (300, 8, 1, 64, 1024, "bf16"),
                                             (1000, 4, 2, 128, 8, "bf16"), (130, 2, 2, 64, 72, "f32"),
                                             (700, 3, 3, 64, 520, "bf16")])
def test_out_proj_ablation_variants(mode, T, G, k, d, D, dtype):
    """The two slot layouts of the ablation table through every kernel path
    (few-token, 128x128-tile, pipelined GEMM, fp32): the hard slots alone,
    W_O with G*k*d rows, and no shared output (passed as NULL, as is the
    hard layout's weight pointer). The weighted layout's slot weights are
    router probabilities, which need not sum to 1 over the selected set.
    The full layout through the same entry point equals gqe_out_proj bit for
    bit."""
    s = synth.make_slot_inputs(T, G, k, d, D, dtype, seed=T + 17)
    p_sel = torch.from_numpy(np.random.default_rng([T, 18]).uniform(0.05, 0.95, (T, G, k)).astype(np.float32))
    g = to_dev(s)
    dims = gqe.gqe_dims.make(1, T, D, G * k, G, k, d, dtype)
    code = {"hard": gqe.GQE_SLOTS_HARD, "weighted": gqe.GQE_SLOTS_WEIGHTED}[mode]
    sw = p_sel.to(DEV) if mode == "weighted" else None
    w_o = g["w_o"][:G * k * d].contiguous()
    y = torch.empty((T, D), dtype=w_o.dtype, device=DEV)
    gqe.gqe_out_proj_variant(dims, code, T, g["o_r"], sw, None, w_o, y)
    y_full = torch.empty_like(y)
    gqe.gqe_out_proj_variant(dims, gqe.GQE_SLOTS_FULL, T, g["o_r"], g["w"], g["o_s"], g["w_o"], y_full)
    torch.cuda.synchronize()
    ref = oracle.out_proj(f64(s["o_r"]), None if sw is None else f64(p_sel), None, f64(w_o), mode=mode)
    assert_close(y, ref, dtype, f"out_proj {mode} T={T}")
    assert torch.equal(y_full, gqe.out_proj(dims, T, g["o_r"], g["w"], g["o_s"], g["w_o"]))


@pytest.mark.parametrize("name", ["main_s2k", "long_s128k", "llama_s8k_skew", "decode_kv64k"])
def test_out_proj_workloads(name):
    """Every output row at the d = 64 workloads (16k and 128k tokens) and at
    decode (16 tokens); 4096 sampled rows of the Llama-shaped one."""
    cfg = synth.workload(name)
    T = cfg.T
    s = synth.make_slot_inputs(T, cfg.G, cfg.k, cfg.d, cfg.D, cfg.dtype, seed=1)
    g = to_dev(s)
    y = gqe.out_proj(dims_of(cfg), T, g["o_r"], g["w"], g["o_s"], g["w_o"])
    torch.cuda.synchronize()
    rows = np.arange(T) if cfg.d <= 64 or T <= 16 else _sample_positions(T, 4096, seed=2)
    w_o = f64(s["w_o"])
    for c0 in range(0, rows.size, 16384):
        r = rows[c0:c0 + 16384]
        ref = oracle.out_proj(f64(s["o_r"][r]), f64(s["w"][r]), f64(s["o_s"][r]), w_o)
        assert_close(y[r], ref, cfg.dtype, f"{name} y rows {r[0]}..{r[-1]} ({r.size})")


# ---------------------------------------------------------------------------
# Whole layer: route -> prefill -> slot assembly + W_O, all on the GPU
# ---------------------------------------------------------------------------

def _layer_gpu(cfg, inp):
    g = to_dev(inp)
    dims = dims_of(cfg)
    r = gqe.route(dims, g["x"], g["w_r"], g["b_r"])
    o_r, o_s = gqe.prefill(dims, g["q"], g["k"], g["v"], r["topk_idx"])
    y = gqe.out_proj(dims, cfg.T, o_r, r["topk_w"], o_s, g["w_o"])
    torch.cuda.synchronize()
    return r, o_r, o_s, y


@pytest.mark.parametrize("cfg", [synth.workload("tiny_f32"),
                                 small_cfg(2, 300, 256, 16, 8, 1, 64),
                                 small_cfg(1, 333, 512, 32, 8, 2, 128, skew=True),
                                 small_cfg(1, 97, 64, 8, 2, 4, 32)], ids=lambda c: f"{c.dtype}-S{c.S}-N{c.N}-k{c.k}")
def test_layer_full(cfg):
    inp = synth.make_prefill_inputs(cfg)
    r, o_r, o_s, y = _layer_gpu(cfg, inp)
    ref = oracle.layer(f64(inp["x"]), f64(inp["w_r"]), f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                       f64(inp["w_o"]), cfg.G, cfg.k, None if inp["b_r"] is None else f64(inp["b_r"]))
    assert np.array_equal(r["topk_idx"].cpu().numpy(), ref["idx"]), "routing differs"
    assert_close(o_r, ref["O_r"], cfg.dtype, "layer O_routed")
    assert_close(o_s, ref["O_s"], cfg.dtype, "layer O_shared")
    assert_close(y, ref["y"], cfg.dtype, "layer y")


@pytest.mark.parametrize("mode", ["hard", "weighted"])
@pytest.mark.parametrize("cfg", [small_cfg(2, 300, 256, 16, 8, 1, 64),
                                 small_cfg(1, 333, 512, 32, 8, 2, 128, skew=True),
                                 small_cfg(1, 130, 256, 4, 2, 1, 32, dtype="f32")],
                         ids=lambda c: f"{c.dtype}-S{c.S}-N{c.N}-k{c.k}")
def test_layer_ablation(cfg, mode):
    """Whole ablation layer on the GPU: route (with the selected p), attend,
    then the hard-slots-only output projection, against the oracle's layer
    with the same layout (weights from slot_weights: p, not the renormalised
    w, so at k = 1 the two layouts give different outputs)."""
    inp = synth.make_prefill_inputs(cfg)
    g = to_dev(inp)
    dims = dims_of(cfg)
    r = gqe.route(dims, g["x"], g["w_r"], g["b_r"], want_p=True)
    o_r, o_s = gqe.prefill(dims, g["q"], g["k"], g["v"], r["topk_idx"])
    T, rows = cfg.T, cfg.G * cfg.k * cfg.d
    w_o = g["w_o"][:rows].contiguous()
    code = {"hard": gqe.GQE_SLOTS_HARD, "weighted": gqe.GQE_SLOTS_WEIGHTED}[mode]
    y = torch.empty((T, cfg.D), dtype=w_o.dtype, device=DEV)
    gqe.gqe_out_proj_variant(dims, code, T, o_r.view(T, cfg.G, cfg.k, cfg.d),
                             r["topk_p"] if mode == "weighted" else None, None, w_o, y)
    torch.cuda.synchronize()
    ref = oracle.layer(f64(inp["x"]), f64(inp["w_r"]), f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                       f64(inp["w_o"][:rows]), cfg.G, cfg.k, None if inp["b_r"] is None else f64(inp["b_r"]),
                       mode=mode)
    assert np.array_equal(r["topk_idx"].cpu().numpy(), ref["idx"]), "routing differs"
    if mode == "weighted":
        assert_close(r["topk_p"], ref["sw"], "f32", "selected p")
        assert np.max(ref["sw"]) < 1.0  # the layout's weights are not the renormalised ones
    assert_close(y, ref["y"], cfg.dtype, f"layer y ({mode})")


def test_layer_main_sampled():
    """The whole layer at the 8 x 2048-token workload: full routing of every
    sequence, and y at 128 sampled positions of each of the 8 sequences."""
    cfg = synth.workload("main_s2k")
    inp = synth.make_prefill_inputs(cfg)
    r, o_r, o_s, y = _layer_gpu(cfg, inp)
    w_o = f64(inp["w_o"])
    for b in range(cfg.B):
        pos = _sample_positions(cfg.S, 128, seed=3 + b)
        z, p, idx, w = oracle.route(f64(inp["x"][b * cfg.S:(b + 1) * cfg.S]), f64(inp["w_r"]), cfg.G, cfg.M,
                                    cfg.k)
        gidx = r["topk_idx"].cpu().numpy()[b * cfg.S:(b + 1) * cfg.S]
        assert np.array_equal(gidx, idx), f"routing differs in sequence {b}"
        ref_r, ref_s = oracle.prefill(f64(inp["q"][b:b + 1]), f64(inp["k"][b:b + 1]), f64(inp["v"][b:b + 1]),
                                      idx.reshape(1, cfg.S, cfg.G, cfg.k), cfg.M, positions=pos)
        yref = oracle.out_proj(ref_r[0].reshape(-1, cfg.G, cfg.k, cfg.d), w[pos], ref_s[0], w_o)
        assert_close(y[b * cfg.S + pos], yref, cfg.dtype, f"main layer y, sequence {b} (sampled)")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_out_of_contract_kv_len_is_contained(dtype):
    """A kv_len outside q_len..S_max breaks the caller's contract; the kernels
    clamp it to the cache, so the other sequences' outputs are still exact
    and nothing outside the caches is read (the violating sequences' outputs
    are unspecified and not checked)."""
    H, G, d, Smax, q_len = 8, 2, 64, 300, 1
    M, k, B = H // G, 2, 4
    rng = np.random.default_rng(77)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, q_len, H + 1, d), dtype=np.float32)).to(tdt)
    kc = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    vc = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    kv_len = np.array([Smax + 1000, 17, -5, 293], dtype=np.int32)
    ok = [1, 3]
    idx = synth.random_selection(B, q_len, G, M, k, 4)
    dims = gqe.gqe_dims.make(B, Smax, 64, H, G, k, d, dtype)
    o_r, o_s = gqe.decode(dims, q_len, q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(kv_len).to(DEV),
                          idx.to(DEV))
    torch.cuda.synchronize()
    ref_r, ref_s = oracle.decode(f64(q)[ok], f64(kc)[ok], f64(vc)[ok], kv_len[ok],
                                 idx.numpy().reshape(B, q_len, G, k)[ok], M)
    assert_close(o_r[ok], ref_r, dtype, "decode beside out-of-contract sequences O_routed")
    assert_close(o_s[ok], ref_s, dtype, "decode beside out-of-contract sequences O_shared")


def test_prefill_out_of_range_index_is_contained():
    """A top-k index outside 0..M-1 breaks the caller's contract; the kernel
    clamps it where it addresses q, so every other row stays exact (the
    corrupted rows' outputs are unspecified and not checked)."""
    cfg = small_cfg(1, 200, 64, 8, 2, 2, 64)
    inp = _prefill_inputs(cfg, False)
    idx = inp["idx"].clone().view(1, 200, cfg.G, cfg.k)
    ref_r, ref_s = oracle.prefill(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), idx.numpy(), cfg.M)
    bad = idx.clone()
    bad[0, 37, 1, 0] = cfg.M + 1000
    bad[0, 150, 0, 1] = -7
    g = to_dev(inp)
    o_r, o_s = gqe.prefill(dims_of(cfg), g["q"], g["k"], g["v"], bad.view(200, cfg.G, cfg.k).to(DEV))
    torch.cuda.synchronize()
    keep = np.ones((1, 200, cfg.G, cfg.k), dtype=bool)
    keep[0, 37, 1, 0] = keep[0, 150, 0, 1] = False
    assert_close(f64(o_r)[keep], ref_r[keep], "bf16", "O_routed beside out-of-range indices")
    assert_close(o_s, ref_s, "bf16", "O_shared beside out-of-range indices")
