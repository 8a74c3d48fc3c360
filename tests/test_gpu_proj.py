"""Parity of the Q/K/V projections (token-compacted Q) with the CPU oracle.

Calls go through the C ABI. Tolerances as for the other kernels (bf16:
max |error| <= 2e-2 and relative Frobenius error <= 1e-2; fp32: 1e-5), with
the bf16 bound scaled by max(1, |ref|) for outputs that exceed 8.
Query rows of unselected heads and cache rows outside the appended ones must
be left bit for bit as they were. The selection comes from the seeded input
generator, so nothing the oracle sees comes from the HIP path.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_query_gqa_amd as gqe
import synth
from test_gpu_parity import DEV, f64
from test_gpu_parity import assert_close as _assert_close_abs


def assert_close(got, ref, dtype, what):
    """As for the other kernels, except that bf16 projections can exceed 8 in
    magnitude, where storing bf16 alone (8 significant bits) rounds by up to
    2^-8 relative: the bound per element is 2e-2 * max(1, |ref|)."""
    if dtype != "bf16":
        return _assert_close_abs(got, ref, dtype, what)
    g = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    scaled = np.abs(g - r) / np.maximum(1.0, np.abs(r))
    worst = float(scaled.max()) if g.size else 0.0
    assert worst <= 2e-2, f"{what}: error {worst:.3e} of max(1, |ref|) > 2e-2"
    _assert_close_abs(np.clip(g, -8, 8), np.clip(r, -8, 8), dtype, what)

pytestmark = pytest.mark.gpu

SENTINEL = 7.0  # exactly representable in bf16 and fp32


def _weights(rng, N, G, d, D, tdt, scale):
    def w(rows):
        return torch.from_numpy(rng.standard_normal((rows, D), dtype=np.float32) * np.float32(scale)).to(tdt)
    return w((N + 1) * d), w(G * d), w(G * d)


def _check_q(q_gpu, Q_ref, dtype, what):
    """Computed rows against the oracle; the rest must still hold the sentinel."""
    got = f64(q_gpu)
    done = ~np.isnan(Q_ref[..., 0])
    assert np.all(got[~done] == SENTINEL), f"{what}: a row of an unselected head was written"
    assert_close(got[done], Q_ref[done], dtype, what)


PREFILL_CASES = [
    # B, S, D, N, G, k, d, dtype, skew
    (2, 300, 256, 8, 2, 1, 64, "bf16", False),    # ragged: 600 tokens, lists of ~300
    (1, 700, 512, 8, 4, 2, 32, "bf16", False),
    (2, 260, 512, 32, 8, 2, 128, "bf16", True),
    (1, 257, 256, 8, 2, 4, 64, "bf16", False),    # k = M: every head
    (1, 200, 256, 8, 8, 1, 64, "bf16", False),    # MHA: G = N
    (3, 90, 192, 4, 1, 2, 32, "bf16", False),     # MQA: G = 1 (M = 4, k = 2)
    (1, 1, 64, 4, 2, 1, 32, "bf16", False),       # one token
    (1, 3000, 256, 16, 4, 1, 64, "bf16", True),   # 1536-token supersteps: shared head and the favoured
                                                  # experts take more than one 512-row pass
    (1, 1000, 128, 6, 3, 1, 64, "bf16", False),   # 384 key/value columns: a half-empty 256-column tile
    (1, 2000, 256, 16, 4, 1, 128, "bf16", True),  # d = 128 head tiles (k32 ring) over several passes
    (1, 128, 256, 4, 2, 1, 32, "f32", False),
    (2, 77, 40, 8, 2, 2, 64, "f32", False),       # fp32 takes any D % 8
]


@pytest.mark.parametrize("B,S,D,N,G,k,d,dtype,skew", PREFILL_CASES)
def test_qkv_proj_matches_oracle(B, S, D, N, G, k, d, dtype, skew):
    M = N // G
    rng = np.random.default_rng(B * 7919 + S * 31 + D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(rng.standard_normal((B, S, D), dtype=np.float32)).to(tdt)
    w_q, w_k, w_v = _weights(rng, N, G, d, D, tdt, 1.0 / np.sqrt(D))
    idx = synth.random_selection(B, S, G, M, k, 5, skew=skew)
    dims = gqe.gqe_dims.make(B, S, D, N, G, k, d, dtype)
    q = torch.full((B, S, N + 1, d), SENTINEL, dtype=tdt, device=DEV)
    print(f"case B={B} S={S} D={D} N={N} G={G} k={k} d={d} {dtype}", flush=True)
    _, kk, vv = gqe.qkv_proj(dims, x.to(DEV), w_q.to(DEV), w_k.to(DEV), w_v.to(DEV), idx.to(DEV), q=q)
    torch.cuda.synchronize()
    Q, K, V = oracle.project(f64(x), f64(w_q), f64(w_k), f64(w_v), idx.numpy().reshape(B, S, G, k), N, G)
    _check_q(q, Q, dtype, "q")
    assert_close(kk, K, dtype, "k")
    assert_close(vv, V, dtype, "v")


DECODE_CASES = [
    # B, q_len, S_max, kv_len per sequence, D, N, G, k, d, dtype
    (3, 1, 40, [1, 17, 40], 256, 8, 2, 1, 64, "bf16"),
    (2, 4, 300, [4, 300], 512, 32, 8, 2, 128, "bf16"),
    (16, 1, 64, list(range(1, 65, 4)), 1024, 32, 8, 2, 128, "bf16"),   # 16 tokens over 16 sequences
    (5, 9, 50, [9, 20, 33, 49, 50], 320, 8, 4, 1, 32, "bf16"),          # 45 tokens: two 32-token chunks
    (2, 3, 10, [3, 10], 64, 4, 2, 2, 32, "f32"),
]


@pytest.mark.parametrize("B,L,Smax,kvl,D,N,G,k,d,dtype", DECODE_CASES)
def test_qkv_proj_decode_matches_oracle(B, L, Smax, kvl, D, N, G, k, d, dtype):
    M = N // G
    rng = np.random.default_rng(B * 131 + L * 17 + D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(rng.standard_normal((B, L, D), dtype=np.float32)).to(tdt)
    w_q, w_k, w_v = _weights(rng, N, G, d, D, tdt, 1.0 / np.sqrt(D))
    kc0 = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    vc0 = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    kv_len = np.array(kvl, dtype=np.int32)
    idx = synth.random_selection(B, L, G, M, k, 6)
    dims = gqe.gqe_dims.make(B, Smax, D, N, G, k, d, dtype)
    q = torch.full((B, L, N + 1, d), SENTINEL, dtype=tdt, device=DEV)
    kc, vc = kc0.to(DEV), vc0.to(DEV)
    print(f"case B={B} q_len={L} Smax={Smax} D={D} N={N} G={G} k={k} d={d} {dtype}", flush=True)
    gqe.gqe_qkv_proj_decode(dims, L, x.to(DEV), w_q.to(DEV), w_k.to(DEV), w_v.to(DEV), idx.to(DEV),
                            torch.from_numpy(kv_len).to(DEV), q, kc, vc)
    torch.cuda.synchronize()
    Q, Kc, Vc = oracle.project_decode(f64(x), f64(w_q), f64(w_k), f64(w_v), idx.numpy().reshape(B, L, G, k),
                                      N, G, kv_len, f64(kc0), f64(vc0))
    _check_q(q, Q, dtype, "q")
    new = np.zeros((B, Smax), dtype=bool)
    for b in range(B):
        new[b, kv_len[b] - L:kv_len[b]] = True
    for name, got, ref, old in (("k cache", kc, Kc, kc0), ("v cache", vc, Vc, vc0)):
        g64 = f64(got)
        keep = ~new[:, None, :, None].repeat(G, 1).repeat(d, 3)
        assert np.array_equal(g64[keep], f64(old)[keep]), f"{name}: a row outside the appended ones changed"
        sel = new[:, None, :].repeat(G, 1)
        assert_close(g64[sel], ref[sel], dtype, name + " appended rows")


@pytest.mark.parametrize("wl,n_sample", [("main_s2k", 512), ("long_s128k", 512), ("llama_s8k_skew", 256)])
def test_qkv_proj_full_size_sampled(wl, n_sample):
    """The full workloads in the launch configuration the benchmark times;
    projections are per token, so sampled tokens are checked against the
    oracle on those tokens alone (first and last token always included)."""
    cfg = synth.workload(wl)
    B, S, D, N, G, k, d, M = cfg.B, cfg.S, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.M
    inp = synth.make_prefill_inputs(cfg, project=False)
    idx = synth.random_selection(B, S, G, M, k, 0, skew=cfg.skew)
    dims = gqe.gqe_dims.from_config(cfg)
    q = torch.full((B, S, N + 1, d), SENTINEL, dtype=torch.bfloat16, device=DEV)
    print(f"workload {wl}", flush=True)
    x = inp["x"].view(B, S, D)
    _, kk, vv = gqe.qkv_proj(dims, x.to(DEV), inp["w_q"].to(DEV), inp["w_k"].to(DEV), inp["w_v"].to(DEV),
                             idx.to(DEV), q=q)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    flat = np.unique(np.concatenate([[0, B * S - 1], rng.choice(B * S, n_sample - 2, replace=False)]))
    xb = f64(x).reshape(B * S, D)[flat][None]
    ib = idx.numpy().reshape(B * S, G, k)[flat][None]
    Q, K, V = oracle.project(xb, f64(inp["w_q"]), f64(inp["w_k"]), f64(inp["w_v"]), ib, N, G)
    bs = np.stack([flat // S, flat % S], 1)
    qs = q.view(B * S, N + 1, d)[torch.from_numpy(flat).to(DEV)]
    _check_q(qs, Q[0], "bf16", f"{wl} q")
    ks = kk[bs[:, 0], :, bs[:, 1]]  # [n, G, d]
    vs = vv[bs[:, 0], :, bs[:, 1]]
    assert_close(ks, K[0].transpose(1, 0, 2), "bf16", f"{wl} k")
    assert_close(vs, V[0].transpose(1, 0, 2), "bf16", f"{wl} v")


def test_qkv_proj_decode_full_size():
    """The decode workload's shape (16 sequences, one new token each, D = 4096,
    32 query heads, k = 2, d = 128) against a short cache."""
    cfg = synth.workload("decode_kv64k")
    B, L, D, N, G, k, d, M = cfg.B, cfg.q_len, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.M
    Smax = 96
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((B, L, D), dtype=np.float32)).to(torch.bfloat16)
    w_q, w_k, w_v = _weights(rng, N, G, d, D, torch.bfloat16, 0.02)
    kc0 = torch.zeros((B, G, Smax, d), dtype=torch.bfloat16)
    kv_len = np.full(B, Smax, dtype=np.int32)
    idx = synth.random_selection(B, L, G, M, k, 0)
    dims = gqe.gqe_dims.make(B, Smax, D, N, G, k, d, "bf16")
    q = torch.full((B, L, N + 1, d), SENTINEL, dtype=torch.bfloat16, device=DEV)
    kc, vc = kc0.to(DEV), kc0.clone().to(DEV)
    gqe.gqe_qkv_proj_decode(dims, L, x.to(DEV), w_q.to(DEV), w_k.to(DEV), w_v.to(DEV), idx.to(DEV),
                            torch.from_numpy(kv_len).to(DEV), q, kc, vc)
    torch.cuda.synchronize()
    Q, Kc, Vc = oracle.project_decode(f64(x), f64(w_q), f64(w_k), f64(w_v), idx.numpy().reshape(B, L, G, k),
                                      N, G, kv_len, f64(kc0), f64(kc0))
    _check_q(q, Q, "bf16", "decode q")
    assert_close(kc[:, :, Smax - 1], Kc[:, :, Smax - 1], "bf16", "decode k")
    assert_close(vc[:, :, Smax - 1], Vc[:, :, Smax - 1], "bf16", "decode v")
    assert torch.count_nonzero(kc[:, :, :Smax - 1]) == 0 and torch.count_nonzero(vc[:, :, :Smax - 1]) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qkv_proj_decode_out_of_contract_kv_len_writes_nothing_outside(dtype):
    """A kv_len that puts appended rows outside 0..S_max-1 breaks the caller's
    contract: those rows are not written (no write lands outside the cache
    or in another sequence), and the in-contract sequences append exactly."""
    B, L, Smax, D, N, G, k, d = 3, 2, 40, 256, 8, 2, 1, 64
    M = N // G
    rng = np.random.default_rng(91)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(rng.standard_normal((B, L, D), dtype=np.float32)).to(tdt)
    w_q, w_k, w_v = _weights(rng, N, G, d, D, tdt, 1.0 / np.sqrt(D))
    kc0 = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    vc0 = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    kv_len = np.array([Smax + 1, 20, 1], dtype=np.int32)  # rows 39, 40 / 18, 19 / -1, 0
    idx = synth.random_selection(B, L, G, M, k, 6)
    dims = gqe.gqe_dims.make(B, Smax, D, N, G, k, d, dtype)
    q = torch.full((B, L, N + 1, d), SENTINEL, dtype=tdt, device=DEV)
    kc, vc = kc0.to(DEV), vc0.to(DEV)
    gqe.gqe_qkv_proj_decode(dims, L, x.to(DEV), w_q.to(DEV), w_k.to(DEV), w_v.to(DEV), idx.to(DEV),
                            torch.from_numpy(kv_len).to(DEV), q, kc, vc)
    torch.cuda.synchronize()
    # projected K/V of every token (the oracle's prefill projection)
    _, K, V = oracle.project(f64(x), f64(w_q), f64(w_k), f64(w_v),
                             idx.numpy().reshape(B, L, G, k), N, G)
    # rows written: sequence 0 row 39 (token 0; its row 40 is skipped),
    # sequence 1 rows 18, 19, sequence 2 row 0 (token 1; its row -1 is skipped)
    written = [(0, 39, 0), (1, 18, 0), (1, 19, 1), (2, 0, 1)]
    new = np.zeros((B, Smax), dtype=bool)
    for b, row, _t in written:
        new[b, row] = True
    for name, got, ref, old in (("k cache", kc, K, kc0), ("v cache", vc, V, vc0)):
        g64 = f64(got)
        keep = ~new[:, None, :, None].repeat(G, 1).repeat(d, 3)
        assert np.array_equal(g64[keep], f64(old)[keep]), f"{name}: a row outside the in-range appends changed"
        for b, row, t in written:
            assert_close(g64[b, :, row], ref[b, :, t], dtype, f"{name} sequence {b} row {row}")
