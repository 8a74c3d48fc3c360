"""Training path on the GPU (through the C ABI) against the CPU oracle:
the forward's row log-sum-exp and the attention backward.

Tolerances. fp32: max |error| <= 1e-5 * max(1, max|ref|), relative Frobenius
error <= 1e-5. bf16 inputs with fp32 accumulation: the backward rounds P and
dS to bf16 for its products (relative error <= 2^-8 each) and rebuilds P from
the forward's lse, whose scores use q*scale*log2(e) rounded to bf16 (relative
error <= 2^-8 of |s|, |s| <= ~8 here); every gradient element is a sum of such
terms, so the bounds are max |error| <= 2e-2 * max(1, max|ref|) and relative
Frobenius error <= 2e-2. The lse itself: |error| <= 2e-2 * max(1, |ref|)
elementwise in bf16, 1e-5 in fp32.
"""
import functools

import numpy as np
import pytest
import torch

import equal_keys
import oracle
import sparse_query_gqa_amd as gqe
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
f64 = synth.to_f64


def _tol(dtype):
    return (2e-2, 2e-2) if dtype == "bf16" else (1e-5, 1e-5)


def assert_grad(got, ref, dtype, what):
    got = f64(got)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    amax, rel = _tol(dtype)
    scale = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    nref = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(got - ref) / max(nref, 1e-300)) if got.size else 0.0
    print(f"{what}: max|err|={err:.3e} (max|ref|={scale:.3e}) rel_fro={fro:.3e}")
    assert err <= amax * scale, f"{what}: max abs error {err:.3e} > {amax * scale:.3e}"
    # A reference whose RMS is below the absolute bound (zero up to rounding,
    # e.g. dq with one visible key) is judged by the absolute bound alone.
    if nref >= np.sqrt(ref.size) * amax:
        assert fro <= rel, f"{what}: relative Frobenius error {fro:.3e} > {rel}"


def _inputs(cfg, seed_do=7):
    inp = synth.make_prefill_inputs(cfg)
    off = (0.25 * torch.arange(cfg.G, dtype=torch.float32)).view(1, cfg.G, 1, 1)
    inp["v"] = (inp["v"].float() + off).to(cfg.torch_dtype)
    inp["idx"] = synth.random_selection(cfg.B, cfg.S, cfg.G, cfg.M, cfg.k, cfg.seed + 5, skew=cfg.skew)
    rng = np.random.default_rng([cfg.seed, seed_do])
    dt = cfg.torch_dtype
    inp["do_r"] = torch.from_numpy(rng.standard_normal((cfg.B, cfg.S, cfg.G, cfg.k, cfg.d), dtype=np.float32)).to(dt)
    inp["do_s"] = torch.from_numpy(rng.standard_normal((cfg.B, cfg.S, cfg.d), dtype=np.float32)).to(dt)
    return inp


def _run(cfg, inp):
    dims = gqe.gqe_dims.from_config(cfg)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o_r, o_s, lse_r, lse_s = gqe.prefill_train(dims, g["q"], g["k"], g["v"], g["idx"])
    dq, dk, dv = gqe.prefill_bwd(dims, g["q"], g["k"], g["v"], g["idx"], o_r, o_s, lse_r, lse_s,
                                 g["do_r"], g["do_s"])
    torch.cuda.synchronize()
    return dict(o_r=o_r, o_s=o_s, lse_r=lse_r, lse_s=lse_s, dq=dq, dk=dk, dv=dv)


def _check(cfg, inp, out, what=""):
    B, S, G, k = cfg.B, cfg.S, cfg.G, cfg.k
    idx = inp["idx"].numpy().reshape(B, S, G, k)
    Q, K, V = f64(inp["q"]), f64(inp["k"]), f64(inp["v"])
    lr, ls = oracle.prefill_lse(Q, K, idx, cfg.M)
    amax = 2e-2 if cfg.dtype == "bf16" else 1e-5
    for got, ref, name in ((out["lse_r"], lr, "lse_r"), (out["lse_s"], ls, "lse_s")):
        e = np.abs(f64(got) - ref) / np.maximum(1.0, np.abs(ref))
        print(f"{what}{name}: max scaled err {float(e.max()):.3e}")
        assert np.all(np.isfinite(f64(got))) and float(e.max()) <= amax, f"{what}{name}"
    dQ, dK, dV = oracle.prefill_bwd(Q, K, V, idx, cfg.M, f64(inp["do_r"]), f64(inp["do_s"]))
    assert_grad(out["dq"], dQ, cfg.dtype, what + "dQ")
    assert_grad(out["dk"], dK, cfg.dtype, what + "dK")
    assert_grad(out["dv"], dV, cfg.dtype, what + "dV")


BWD_CASES = [
    # B, S, D, N, G, k, d, dtype
    (1, 1, 64, 4, 2, 1, 32, "f32"),
    (1, 128, 256, 4, 2, 1, 32, "f32"),  # the tiny fp32 layer's shape
    (2, 77, 64, 8, 2, 3, 64, "f32"),
    (1, 150, 64, 6, 6, 1, 128, "f32"),
    (1, 1, 64, 4, 2, 1, 64, "bf16"),
    (1, 7, 64, 8, 1, 2, 64, "bf16"),
    (2, 300, 128, 16, 8, 1, 64, "bf16"),
    (1, 517, 128, 32, 8, 2, 128, "bf16"),
    (3, 200, 64, 8, 4, 2, 32, "bf16"),
    (1, 129, 64, 8, 8, 1, 64, "bf16"),
    (1, 64, 64, 16, 4, 4, 64, "bf16"),
    (2, 100, 64, 8, 8, 1, 128, "bf16"),  # MHA (M = 1)
    (1, 300, 64, 4, 1, 4, 128, "bf16"),  # dense MQA (G = 1, k = M)
    (1, 333, 64, 8, 8, 1, 64, "f32"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_bwd_small(case):
    B, S, D, N, G, k, d, dtype = case
    cfg = synth.GQEConfig("case", B=B, S=S, D=D, N=N, G=G, k=k, d=d, dtype=dtype, seed=3)
    inp = _inputs(cfg)
    print(f"case {case}", flush=True)
    _check(cfg, inp, _run(cfg, inp))


def test_prefill_train_forward_matches_inference():
    """The training forward writes the same outputs as the inference call."""
    cfg = synth.GQEConfig("case", B=2, S=300, D=128, N=16, G=8, k=1, d=64, dtype="bf16", seed=4)
    inp = _inputs(cfg)
    dims = gqe.gqe_dims.from_config(cfg)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    a_r, a_s = gqe.prefill(dims, g["q"], g["k"], g["v"], g["idx"])
    b_r, b_s, _, _ = gqe.prefill_train(dims, g["q"], g["k"], g["v"], g["idx"])
    assert torch.equal(a_r, b_r) and torch.equal(a_s, b_s)


def test_prefill_bwd_deterministic():
    cfg = synth.GQEConfig("case", B=1, S=517, D=128, N=32, G=8, k=2, d=128, dtype="bf16", seed=5)
    inp = _inputs(cfg)
    a = _run(cfg, inp)
    b = _run(cfg, inp)
    for n in ("dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n


def test_prefill_bwd_skewed_routing():
    """One expert per group favoured 3:1: uneven heads, same sums."""
    cfg = synth.GQEConfig("case", B=2, S=250, D=128, N=32, G=8, k=2, d=128, dtype="bf16", seed=6, skew=True)
    inp = _inputs(cfg)
    _check(cfg, inp, _run(cfg, inp))


def test_prefill_bwd_main_workload():
    """The 2k-token bf16 layer (batch 8, N=16, G=8, k=1, d=64), in the launch
    configuration the benchmark times; the oracle checks sequences 0 and 7
    in full."""
    cfg = synth.workload("main_s2k")
    inp = _inputs(cfg)
    out = _run(cfg, inp)
    for b in (0, cfg.B - 1):
        sub = synth.GQEConfig("case", B=1, S=cfg.S, D=cfg.D, N=cfg.N, G=cfg.G, k=cfg.k, d=cfg.d, dtype=cfg.dtype,
                              seed=cfg.seed)
        one = {n: inp[n][b:b + 1] for n in ("q", "k", "v", "do_r", "do_s")}
        one["idx"] = inp["idx"].view(cfg.B, cfg.S, cfg.G, cfg.k)[b:b + 1].reshape(cfg.S, cfg.G, cfg.k)
        got = {n: out[n][b:b + 1] for n in ("lse_r", "lse_s", "dq", "dk", "dv")}
        _check(sub, one, got, what=f"b={b} ")


@functools.lru_cache(maxsize=1)
def _long_case():
    cfg = synth.workload("long_s128k")
    return cfg, _inputs(cfg)


def _rows(t, dim, pos):
    return t.index_select(dim, torch.as_tensor(pos, dtype=torch.long, device=t.device))


def test_prefill_bwd_long_workload_sampled():
    """The 128k-token bf16 layer (batch 1, N=16, G=8, k=1, d=64) in the launch
    configuration the benchmark times. The oracle takes 15 rows spread over
    the sequence and the last 64: the forward's lse and every head's dQ at
    those rows, and dK, dV of the last 64 keys of every KV head, which no
    earlier row can see."""
    cfg, inp = _long_case()
    out = _run(cfg, inp)
    S, tail = cfg.S, 64
    rng = np.random.default_rng(11)
    spread = rng.choice(np.arange(1, S - tail), size=14, replace=False)
    pos = np.sort(np.concatenate([[0], spread, np.arange(S - tail, S)]))
    print(f"long_s128k rows {pos[:15].tolist()} + last {tail}", flush=True)
    idx = inp["idx"].numpy().reshape(cfg.B, S, cfg.G, cfg.k)
    Q, K, V = f64(inp["q"]), f64(inp["k"]), f64(inp["v"])
    lr, ls = oracle.prefill_lse(Q, K, idx, cfg.M, positions=pos)
    for got, ref, name in ((_rows(out["lse_r"], 1, pos), lr, "lse_r"), (_rows(out["lse_s"], 1, pos), ls, "lse_s")):
        e = np.abs(f64(got) - ref) / np.maximum(1.0, np.abs(ref))
        print(f"{name}: max scaled err {float(e.max()):.3e}")
        assert np.all(np.isfinite(f64(got))) and float(e.max()) <= 2e-2, name
    dQ, dK, dV = oracle.prefill_bwd(Q, K, V, idx, cfg.M, f64(inp["do_r"]), f64(inp["do_s"]), positions=pos)
    assert_grad(_rows(out["dq"], 1, pos), dQ, cfg.dtype, "dQ (sampled rows)")
    assert_grad(out["dk"][:, :, S - tail:], dK[:, :, S - tail:], cfg.dtype, "dK (last keys)")
    assert_grad(out["dv"][:, :, S - tail:], dV[:, :, S - tail:], cfg.dtype, "dV (last keys)")


def test_prefill_bwd_long_workload_equal_keys():
    """The same layer with every key of a KV head set to its first key: each
    softmax row is uniform over the visible keys, and the lse of every row and
    the dK, dV of every key have closed forms (equal_keys), checked in full.
    dQ is zero in exact arithmetic; what the kernel returns is rounding of a
    sum whose terms cancel, chiefly from delta_i = dO_i . o_i taken with the
    stored bf16 o_i, so each element is held to 2e-2 of the size of those
    terms, scale * |k_c| * sum_c' |dO_ic'| |o_ic'| (at least 1). The kernels
    leave the dQ rows of unselected heads unwritten, so they keep the zeros
    the binding allocates."""
    cfg, inp = _long_case()
    B, S, G, M, k, N, d = cfg.B, cfg.S, cfg.G, cfg.M, cfg.k, cfg.N, cfg.d
    e = dict(inp)
    e["k"] = inp["k"][:, :, :1].expand(-1, -1, S, -1).contiguous()
    out = _run(cfg, e)
    idx = inp["idx"].view(B, S, G, k).long()
    rows = torch.arange(S)
    lse_r, lse_s = f64(out["lse_r"]), f64(out["lse_s"])
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        dK = np.zeros((G, S, d))
        dV = np.zeros((G, S, d))
        used = torch.zeros((S, N + 1), dtype=torch.bool)
        used[:, N] = True
        dqb = out["dq"][b].cpu()
        worst = 0.0

        def check_dq(heads, key, dO, o):
            nonlocal worst
            got = f64(dqb[rows, heads])
            tol = 2e-2 * np.maximum(1.0, scale * np.abs(key)[None, :] * np.sum(np.abs(dO) * np.abs(o), 1)[:, None])
            worst = max(worst, float(np.max(np.abs(got) / tol)))
            assert np.all(np.abs(got) <= tol), f"b={b} dQ of heads {heads[:4].tolist()}..."

        for g in range(G):
            key = f64(e["k"][b, g, 0])
            for j in range(k):
                heads = g * M + idx[b, :, g, j]
                used[rows, heads] = True
                dO = f64(inp["do_r"][b, :, g, j])
                lse, o, dk, dv = equal_keys.stream(f64(inp["q"][b, rows, heads]), dO, f64(inp["v"][b, g]), key)
                dK[g] += dk
                dV[g] += dv
                err = np.abs(lse_r[b, :, g, j] - lse) / np.maximum(1.0, np.abs(lse))
                assert float(err.max()) <= 2e-2, f"lse_r b={b} g={g} j={j}: {float(err.max()):.3e}"
                check_dq(heads, key, dO, o)
        key = f64(e["k"][b, 0, 0])
        dO = f64(inp["do_s"][b])
        lse, o, dk, dv = equal_keys.stream(f64(inp["q"][b, :, N]), dO, f64(inp["v"][b, 0]), key)
        dK[0] += dk
        dV[0] += dv
        err = np.abs(lse_s[b] - lse) / np.maximum(1.0, np.abs(lse))
        assert float(err.max()) <= 2e-2, f"lse_s b={b}: {float(err.max()):.3e}"
        check_dq(torch.full((S,), N), key, dO, o)
        print(f"b={b} dQ: largest |dQ| / bound = {worst:.3e}")
        assert_grad(out["dk"][b], dK, cfg.dtype, f"b={b} dK (every key)")
        assert_grad(out["dv"][b], dV, cfg.dtype, f"b={b} dV (every key)")
        assert not bool(dqb[~used].any()), f"b={b}: dQ rows of unselected heads were written"
