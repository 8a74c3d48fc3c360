"""Backward of the output projection and of the router on the GPU (through
the C ABI) against the CPU oracle.

Tolerances. fp32: max |error| <= 1e-5 * max(1, max|ref|), relative Frobenius
error <= 1e-5. bf16: the products take bf16 operands with fp32 accumulation;
the slot vector's obar and the router's dz are rounded to bf16 before their
weight-gradient products (relative error <= 2^-8 per term) and the bf16
outputs are rounded once more, so max |error| <= 2e-2 * max(1, max|ref|) and
relative Frobenius error <= 1e-2. Quantities the kernels keep in fp32 (dw,
dz, db_r, the balance loss) are held to 1e-4 relative in both dtypes.
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
MODES = {"full": gqe.GQE_SLOTS_FULL, "hard": gqe.GQE_SLOTS_HARD, "weighted": gqe.GQE_SLOTS_WEIGHTED}


def assert_close(got, ref, tol, what, rel=None):
    got = f64(got)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    scale = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    nref = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(got - ref) / max(nref, 1e-300)) if got.size else 0.0
    print(f"{what}: max|err|={err:.3e} (max|ref|={scale:.3e}) rel_fro={fro:.3e}")
    assert err <= tol * scale, f"{what}: max abs error {err:.3e} > {tol * scale:.3e}"
    if rel is not None and nref >= np.sqrt(ref.size) * tol:
        assert fro <= rel, f"{what}: relative Frobenius error {fro:.3e} > {rel}"


def _tols(dtype):
    return (2e-2, 1e-2) if dtype == "bf16" else (1e-5, 1e-5)


def _tensor(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt)


OUT_CASES = [
    # T, G, k, d, D, dtype
    (1, 2, 1, 32, 64, "f32"),
    (37, 2, 2, 64, 96, "f32"),
    (129, 4, 1, 128, 64, "f32"),
    (1, 2, 1, 64, 64, "bf16"),
    (37, 8, 1, 64, 1024, "bf16"),
    (300, 2, 2, 32, 96, "bf16"),
    (1000, 8, 2, 128, 256, "bf16"),
    (3000, 4, 1, 64, 128, "bf16"),
]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("case", OUT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_out_proj_bwd(case, mode):
    T, G, k, d, D, dtype = case
    rng = np.random.default_rng([T, G, k, d, D])
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    O_r = _tensor(rng.standard_normal((T, G, k, d)), dt)
    wraw = rng.random((T, G, k)) + 0.1
    # slot weights: renormalised w for the full layout, router probabilities
    # (not summing to 1 over the selected set) for the weighted one, none for
    # the hard one; the ablation layouts take no shared output
    if mode == "full":
        w = torch.from_numpy((wraw / wraw.sum(-1, keepdims=True)).astype(np.float32))
    else:
        w = torch.from_numpy((wraw / (wraw.sum(-1, keepdims=True) + 0.5)).astype(np.float32))
    O_s = _tensor(rng.standard_normal((T, d)), dt)
    rows = (G * k + (2 if mode == "full" else 0)) * d
    W_O = _tensor(rng.standard_normal((rows, D)) * 0.05, dt)
    dy = _tensor(rng.standard_normal((T, D)), dt)
    dims = gqe.gqe_dims.make(1, T, D, G * max(k, 2), G, k, d, dtype)
    full = mode == "full"
    do_r, dw, do_s, dw_o = gqe.out_proj_bwd(dims, T, O_r.to(DEV), None if mode == "hard" else w.to(DEV),
                                            O_s.to(DEV) if full else None, W_O.to(DEV), dy.to(DEV),
                                            mode=MODES[mode])
    torch.cuda.synchronize()
    ref = oracle.out_proj_bwd(f64(O_r), None if mode == "hard" else f64(w), f64(O_s) if full else None,
                              f64(W_O), f64(dy), mode=mode)
    tol, rel = _tols(dtype)
    assert_close(do_r, ref[0], tol, "dO_r", rel)
    assert_close(dw, ref[1], 1e-4, "dw", 1e-4)
    assert_close(do_s, ref[2], tol, "dO_s", rel)
    assert_close(dw_o, ref[3], tol, "dW_O", rel)


@pytest.mark.parametrize("name", ["main_s2k", "long_s128k"])
def test_out_proj_bwd_workload(name):
    """The bf16 layers' shapes (2k tokens x 8 sequences and 128k tokens, G*k
    = 8 slots of d = 64, D = 1024), the second in the launch configuration
    the benchmark times: every output in full, the weight gradient summing
    over all 16384 or 131072 tokens."""
    cfg = synth.workload(name)
    T, G, k, d, D = cfg.T, cfg.G, cfg.k, cfg.d, cfg.D
    rng = np.random.default_rng(9)
    O_r = _tensor(rng.standard_normal((T, G, k, d)), torch.bfloat16)
    w = torch.ones((T, G, k), dtype=torch.float32)
    O_s = _tensor(rng.standard_normal((T, d)), torch.bfloat16)
    W_O = _tensor(rng.standard_normal(((G * k + 2) * d, D)) * 0.02, torch.bfloat16)
    dy = _tensor(rng.standard_normal((T, D)), torch.bfloat16)
    dims = gqe.gqe_dims.from_config(cfg)
    do_r, dw, do_s, dw_o = gqe.out_proj_bwd(dims, T, O_r.to(DEV), w.to(DEV), O_s.to(DEV), W_O.to(DEV), dy.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.out_proj_bwd(f64(O_r), f64(w), f64(O_s), f64(W_O), f64(dy))
    assert_close(do_r, ref[0], 2e-2, "dO_r", 1e-2)
    assert_close(dw, ref[1], 1e-4, "dw", 1e-4)
    assert_close(do_s, ref[2], 2e-2, "dO_s", 1e-2)
    assert_close(dw_o, ref[3], 2e-2, "dW_O", 1e-2)


ROUTE_CASES = [
    # T, D, G, M, k, dtype, aux
    (1, 64, 2, 2, 1, "f32", 0.0),
    (77, 40, 3, 4, 2, "f32", 0.01),
    (200, 256, 8, 32, 5, "f32", 0.1),
    (1, 64, 2, 2, 1, "bf16", 0.0),
    (130, 64, 8, 2, 1, "bf16", 0.01),
    (333, 96, 2, 32, 3, "bf16", 0.05),
    (2500, 128, 16, 16, 3, "bf16", 0.01),
]


@pytest.mark.parametrize("wrt", ["w", "p"])
@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_route_bwd(case, wrt):
    """dw is the gradient of the renormalised weights (wrt w, the full
    layout) or of the selected probabilities (wrt p, the weighted
    ablation layout)."""
    T, D, G, M, k, dtype, aux = case
    rng = np.random.default_rng([T, D, G, M, k])
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = _tensor(rng.standard_normal((T, D)), dt)
    w_r = _tensor(rng.standard_normal((G * M, D)) * 0.1, dt)
    # logits and selection from the oracle (fp32-rounded logits, as gqe_route stores them)
    z = oracle.route_logits(f64(x), f64(w_r), G, M).astype(np.float32)
    _, idx, _ = oracle.route_select(z.astype(np.float64), k)
    dw = rng.standard_normal((T, G, k)).astype(np.float32)
    dims = gqe.gqe_dims.make(1, T, D, G * M, G, k, 32, dtype)
    kind = gqe.GQE_WEIGHTS_RENORM if wrt == "w" else gqe.GQE_WEIGHTS_PROB
    out = gqe.route_bwd(dims, x.to(DEV), w_r.to(DEV), torch.from_numpy(z).to(DEV),
                        torch.from_numpy(idx.astype(np.int32)).to(DEV), torch.from_numpy(dw).to(DEV), aux_coef=aux,
                        weights=kind)
    torch.cuda.synchronize()
    dz, dW_r, db_r, dx = oracle.route_bwd(f64(x), f64(w_r), z.astype(np.float64), idx, dw.astype(np.float64),
                                          G, M, aux_coef=aux, wrt=wrt)
    tol, rel = _tols(dtype)
    assert_close(out["dz"], dz, 1e-4, "dz", 1e-4)
    assert_close(out["db_router"], db_r, 1e-4, "db_r", 1e-4)
    assert_close(out["dw_router"], dW_r, tol, "dW_r", rel)
    assert_close(out["dx"], dx, tol, "dx", rel)
    loss = oracle.load_balance_loss(z.astype(np.float64), idx, M, aux)
    got = float(out["aux_loss"].cpu()[0])
    print(f"aux loss {got:.6e} vs {loss:.6e}")
    assert abs(got - loss) <= 1e-5 * max(1.0, abs(loss))


@pytest.mark.parametrize("name", ["main_s2k", "long_s128k"])
def test_route_bwd_workload(name):
    """The router backward at the bf16 layers' sizes (G = 8 groups of M = 2
    experts, top-1, D = 1024) with the balance loss, the 128k-token one in the
    launch configuration the benchmark times; every output in full."""
    cfg = synth.workload(name)
    T, D, G, M, k = cfg.T, cfg.D, cfg.G, cfg.M, cfg.k
    rng = np.random.default_rng(13)
    x = _tensor(rng.standard_normal((T, D)), torch.bfloat16)
    w_r = _tensor(rng.standard_normal((G * M, D)) * 0.02, torch.bfloat16)
    z = oracle.route_logits(f64(x), f64(w_r), G, M).astype(np.float32)
    _, idx, _ = oracle.route_select(z.astype(np.float64), k)
    dw = rng.standard_normal((T, G, k)).astype(np.float32)
    dims = gqe.gqe_dims.from_config(cfg)
    out = gqe.route_bwd(dims, x.to(DEV), w_r.to(DEV), torch.from_numpy(z).to(DEV),
                        torch.from_numpy(idx.astype(np.int32)).to(DEV), torch.from_numpy(dw).to(DEV), aux_coef=0.01)
    torch.cuda.synchronize()
    dz, dW_r, db_r, dx = oracle.route_bwd(f64(x), f64(w_r), z.astype(np.float64), idx, dw.astype(np.float64),
                                          G, M, aux_coef=0.01)
    # With top-1 the renormalised weight is 1 whatever the logits, so only the
    # balance loss reaches the router and every gradient is of its (small)
    # size: the bounds are relative to the largest reference element.
    for name, ref, tol in (("dz", dz, 1e-4), ("db_router", db_r, 1e-4), ("dw_router", dW_r, 2e-2),
                           ("dx", dx, 2e-2)):
        got = f64(out[name])
        amax = float(np.max(np.abs(ref)))
        err = float(np.max(np.abs(got - ref)))
        fro = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        print(f"{name}: max|err|={err:.3e} (max|ref|={amax:.3e}) rel_fro={fro:.3e}")
        assert amax > 0 and err <= tol * amax and fro <= tol / 2, name
    loss = oracle.load_balance_loss(z.astype(np.float64), idx, M, 0.01)
    got = float(out["aux_loss"].cpu()[0])
    assert abs(got - loss) <= 1e-5 * max(1.0, abs(loss)), (got, loss)


def test_route_bwd_deterministic():
    T, D, G, M, k = 5000, 128, 8, 4, 2
    rng = np.random.default_rng(3)
    x = _tensor(rng.standard_normal((T, D)), torch.bfloat16).to(DEV)
    w_r = _tensor(rng.standard_normal((G * M, D)) * 0.1, torch.bfloat16).to(DEV)
    z = torch.from_numpy(rng.standard_normal((T, G, M)).astype(np.float32)).to(DEV)
    idx = torch.from_numpy(np.sort(np.argsort(-z.cpu().numpy(), -1)[..., :k], -1).astype(np.int32)).to(DEV)
    dw = torch.from_numpy(rng.standard_normal((T, G, k)).astype(np.float32)).to(DEV)
    dims = gqe.gqe_dims.make(1, T, D, G * M, G, k, 32, "bf16")
    a = gqe.route_bwd(dims, x, w_r, z, idx, dw, aux_coef=0.01)
    b = gqe.route_bwd(dims, x, w_r, z, idx, dw, aux_coef=0.01)
    for n in a:
        assert torch.equal(a[n], b[n]), n
