"""The layer's entry points under HIP graph capture.

None of the library's launches allocates device memory or clears it with a
memset, so a caller can capture them. These tests capture a whole prefill
layer (gqe_route with its token lists, gqe_qkv_proj, gqe_attn_prefill,
gqe_out_proj) and a whole decode step (gqe_route, gqe_qkv_proj_decode with
the K/V append, gqe_attn_decode, gqe_out_proj) into one graph each. The
graph is replayed several times with eager calls and synchronisations in
between, and with new values copied into its input tensors; every replay
must equal the eager result bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import sparse_query_gqa_amd as gqe
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _prefill_layer(dims, st):
    """Route -> projections -> attention -> output projection into st's outputs."""
    T, G, k, d = dims.B * dims.S, dims.G, dims.k, dims.d
    gqe.gqe_route(dims, st["x"], st["w_r"], st["b_r"], None, st["idx"], st["w"], st["list_off"],
                  st["list_tok"], st["r_ws"])
    gqe.gqe_qkv_proj(dims, st["x"].view(dims.B, dims.S, dims.D), st["w_q"], st["w_k"], st["w_v"], st["idx"],
                     st["q"], st["k"], st["v"])
    gqe.gqe_attn_prefill(dims, st["q"], st["k"], st["v"], st["idx"], st["o_r"], st["o_s"])
    gqe.gqe_out_proj(dims, T, st["o_r"].view(T, G, k, d), st["w"], st["o_s"].view(T, d), st["w_o"], st["y"])


def _prefill_state(cfg, inp):
    dims = gqe.gqe_dims.from_config(cfg)
    B, S, D, N, G, k, d, M, T = cfg.B, cfg.S, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.M, cfg.T
    dt = cfg.torch_dtype
    st = {n: inp[n].to(DEV) for n in ("x", "w_r", "w_q", "w_k", "w_v", "w_o")}
    st["b_r"] = None if inp["b_r"] is None else inp["b_r"].to(DEV)
    st.update(idx=torch.empty((T, G, k), dtype=torch.int32, device=DEV),
              w=torch.empty((T, G, k), dtype=torch.float32, device=DEV),
              list_off=torch.empty((B, G, M + 1), dtype=torch.int32, device=DEV),
              list_tok=torch.empty((B, G, k * S), dtype=torch.int32, device=DEV),
              r_ws=torch.empty((max(gqe.gqe_route_workspace_bytes(dims), 16),), dtype=torch.uint8, device=DEV),
              q=torch.zeros((B, S, N + 1, d), dtype=dt, device=DEV),
              k=torch.empty((B, G, S, d), dtype=dt, device=DEV),
              v=torch.empty((B, G, S, d), dtype=dt, device=DEV),
              o_r=torch.empty((B, S, G, k, d), dtype=dt, device=DEV),
              o_s=torch.empty((B, S, d), dtype=dt, device=DEV),
              y=torch.empty((T, D), dtype=dt, device=DEV))
    return dims, st


OUTS_PREFILL = ("idx", "w", "list_off", "list_tok", "q", "k", "v", "o_r", "o_s", "y")


def _snapshot(st, names):
    return {n: st[n].clone() for n in names}


def _capture(fn):
    """Warm up on a side stream (as torch asks before capture), then capture fn."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _check_equal(got, ref, what):
    for n, t in ref.items():
        assert torch.equal(st_view(got[n]), st_view(t)), f"{what}: {n} differs from the eager result"


def st_view(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("cfg", [synth.GQEConfig("case", B=2, S=700, D=256, N=16, G=8, k=1, d=64),
                                 synth.GQEConfig("case", B=1, S=333, D=512, N=32, G=8, k=2, d=128, skew=True)],
                         ids=lambda c: f"S{c.S}-d{c.d}-k{c.k}")
def test_prefill_layer_graph_replay(cfg):
    dims, st = _prefill_state(cfg, synth.make_prefill_inputs(cfg, project=False))
    print(f"case prefill B={cfg.B} S={cfg.S} D={cfg.D} N={cfg.N} G={cfg.G} k={cfg.k} d={cfg.d}", flush=True)
    _prefill_layer(dims, st)
    torch.cuda.synchronize()
    eager = _snapshot(st, OUTS_PREFILL)
    g = _capture(lambda: _prefill_layer(dims, st))
    # a second input set, copied into the graph's input tensors between replays
    other = synth.make_prefill_inputs(cfg.replace(seed=cfg.seed + 5), project=False)
    x0 = st["x"].clone()
    for rep in range(4):
        use_other = rep % 2 == 1
        st["x"].copy_(other["x"].to(DEV) if use_other else x0)
        if use_other:
            st["q"].zero_()  # the rows of unselected heads are left as they were
            _prefill_layer(dims, st)  # eager on the new input, then clear the outputs
            torch.cuda.synchronize()
            want = _snapshot(st, OUTS_PREFILL)
        else:
            want = eager
        for n in ("o_r", "o_s", "y"):
            st[n].fill_(float("nan"))
        st["q"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check_equal(st, want, f"replay {rep} ({'second' if use_other else 'first'} input)")


def _decode_step(dims, rdims, st):
    L, T = st["q_len"], st["T"]
    G, k, d = dims.G, dims.k, dims.d
    gqe.gqe_route(rdims, st["x"].view(T, dims.D), st["w_r"], st["b_r"], None, st["idx"], st["w"], None, None,
                  None)
    gqe.gqe_qkv_proj_decode(dims, L, st["x"], st["w_q"], st["w_k"], st["w_v"], st["idx"], st["kv_len"], st["q"],
                            st["kc"], st["vc"])
    gqe.gqe_attn_decode(dims, L, st["q"], st["kc"], st["vc"], st["kv_len"], st["idx"], st["o_r"], st["o_s"],
                        st["ws"])
    gqe.gqe_out_proj(dims, T, st["o_r"].view(T, G, k, d), st["w"], st["o_s"].view(T, d), st["w_o"], st["y"])


@pytest.mark.parametrize("q_len", [1, 3])
def test_decode_step_graph_replay(q_len):
    cfg = synth.GQEConfig("case", B=4, S=3000, D=512, N=32, G=8, k=2, d=128, mode="decode", q_len=q_len,
                          kv_len=2500)
    print(f"case decode B={cfg.B} q_len={q_len} kv_len={cfg.kv_len} Smax={cfg.S}", flush=True)
    inp = synth.make_decode_inputs(cfg)
    dims = gqe.gqe_dims.from_config(cfg)
    rdims = gqe.gqe_dims.make(cfg.B, q_len, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.dtype)
    B, D, N, G, k, d, T = cfg.B, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.T
    dt = cfg.torch_dtype
    st = {n: inp[n].to(DEV) for n in ("w_r", "w_q", "w_k", "w_v", "w_o", "kv_len")}
    st["b_r"] = None if inp["b_r"] is None else inp["b_r"].to(DEV)
    st["x"] = inp["x"].to(DEV).view(B, q_len, D)
    st["kc"], st["vc"] = inp["k"].to(DEV), inp["v"].to(DEV)
    st.update(q_len=q_len, T=T,
              idx=torch.empty((T, G, k), dtype=torch.int32, device=DEV),
              w=torch.empty((T, G, k), dtype=torch.float32, device=DEV),
              q=torch.zeros((B, q_len, N + 1, d), dtype=dt, device=DEV),
              ws=gqe.decode_workspace(dims, q_len, DEV),
              o_r=torch.empty((B, q_len, G, k, d), dtype=dt, device=DEV),
              o_s=torch.empty((B, q_len, d), dtype=dt, device=DEV),
              y=torch.empty((T, D), dtype=dt, device=DEV))
    names = ("idx", "w", "q", "kc", "vc", "o_r", "o_s", "y")
    _decode_step(dims, rdims, st)
    torch.cuda.synchronize()
    eager = _snapshot(st, names)
    g = _capture(lambda: _decode_step(dims, rdims, st))
    rng = np.random.default_rng(q_len)
    x0 = st["x"].clone()
    x1 = torch.from_numpy(rng.standard_normal((B, q_len, D), dtype=np.float32)).to(dt).to(DEV)
    for rep in range(4):
        use_other = rep % 2 == 1
        st["x"].copy_(x1 if use_other else x0)
        if use_other:
            st["q"].zero_()
            _decode_step(dims, rdims, st)
            torch.cuda.synchronize()
            want = _snapshot(st, names)
        else:
            want = eager
        for n in ("o_r", "o_s", "y"):
            st[n].fill_(float("nan"))
        st["q"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check_equal(st, want, f"replay {rep} ({'second' if use_other else 'first'} input)")


def test_two_streams_concurrently():
    """Two prefill layers of different shapes launched on two streams at once
    give the same bits as when they run one after the other: the entry points
    keep no state between calls (each call's scratch is the caller's), so
    concurrent calls on one device do not interfere."""
    cfgs = [synth.GQEConfig("case", B=2, S=700, D=256, N=16, G=8, k=1, d=64),
            synth.GQEConfig("case", B=1, S=333, D=512, N=32, G=8, k=2, d=128, skew=True, seed=3)]
    states = [_prefill_state(c, synth.make_prefill_inputs(c, project=False)) for c in cfgs]
    seq = []
    for dims, st in states:
        _prefill_layer(dims, st)
        torch.cuda.synchronize()
        seq.append(_snapshot(st, OUTS_PREFILL))
    for _, st in states:
        for n in ("o_r", "o_s", "y"):
            st[n].fill_(float("nan"))
        st["q"].zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for s, (dims, st) in zip(streams, states):
            with torch.cuda.stream(s):
                _prefill_layer(dims, st)
        torch.cuda.synchronize()
        for i, (_, st) in enumerate(states):
            _check_equal(st, seq[i], f"concurrent run {rep}, layer {i}")
