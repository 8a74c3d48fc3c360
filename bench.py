"""Benchmark of the GQE layer's hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step runs both halves of the hot path on seeded synthetic inputs that
are resident in HBM before timing starts:
  * prefill (long context): gqe_route (+ token lists) -> gqe_attn_prefill ->
    gqe_out_proj on B=1, S=131072, D=1024, N=16, G=8, k=1, d=64, bf16;
  * decode (long KV): gqe_route -> gqe_attn_decode -> gqe_out_proj for 16
    sequences x 1 new token against 65536 cached keys each (G=8, d=128, k=2).
All launches go to torch's current stream; HIP events on that stream bracket
every call, so per-call durations are measured live.

`value` is the prefill path's algorithmic throughput (router + attention +
output-projection FLOP / its measured time). `decode` reports the decode
path's KV-cache bytes per second. `roofline` is for the dominant kernel,
the prefill attention: attention FLOP per launch / its average launch
duration against the bf16 dense MFMA peak. `cpu_baseline` times the CPU
oracle on a bounded sample of the same prefill workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_query_gqa_amd as gqe  # noqa: E402
import synth  # noqa: E402

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA, published
PEAK_HBM_BPS = 8.0e12      # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")


def prefill_path_flops(cfg) -> dict:
    """Algorithmic FLOP of one prefill-path call (matmul FLOP only)."""
    T, D, G, M, k, d = cfg.T, cfg.D, cfg.G, cfg.M, cfg.k, cfg.d
    attn = 4 * d * (G * k + 1) * cfg.B * cfg.S * (cfg.S + 1) // 2
    router = 2 * T * D * G * M
    proj = 2 * T * (G * k + 2) * d * D + 2 * T * G * k * d  # W_O GEMM + weighted sum
    return dict(attention=attn, router=router, out_proj=proj, total=attn + router + proj)


def projection_flops(T: int, D: int, G: int, k: int, d: int) -> int:
    """Matmul FLOP of the token-compacted projections: 2*D per output value,
    (G*k+1)*d query columns (selected heads + shared head) and 2*G*d
    key/value columns per token."""
    return 2 * T * D * ((G * k + 1) * d + 2 * G * d)


def decode_kv_bytes(cfg) -> int:
    """KV-cache bytes one decode call must read: 2*B*G*kv_len*d*b (one layer)."""
    return 2 * cfg.B * cfg.G * cfg.kv_len * cfg.d * 2


def source_sha(name: str) -> str:
    """Hash of a kernel source together with the internal headers (shared
    device helpers and tile geometry), so that a change to any of them
    retires old counters."""
    h = hashlib.sha256()
    for n in (name, "gqe_internal.h", "prefill_tiles.h"):
        with open(os.path.join(ROOT, "sparse_query_gqa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_file: str, summary: str):
    """HBM bytes per launch from a committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"traffic_bytes_per_launch=(\d+)\s+source_sha=([0-9a-f]+)", txt)
    if not m or m.group(2) != source_sha(kernel_file):
        return None
    return int(m.group(1))


def routing_stats(dims, cfg, x, w_r, b_r, logits, list_off) -> dict:
    """Realised routing of one prefill: per-(group, expert) token counts
    summed over the sequences (from gqe_route's lists), their share of each
    group's T*k selections, and the near ties: (token, group) pairs whose
    top-k margin in the emitted fp32 logits is within twice the fp32 logit
    error bound 1e-5 * (1 + sum_j |x_j w_j|), where a different summation
    order could change the selection. Reporting only (torch on the device)."""
    T, G, M, k = cfg.T, cfg.G, cfg.M, cfg.k
    counts = torch.diff(list_off, dim=-1).sum(0).cpu().numpy()  # [G, M]
    share = counts / float(T * k)
    near = 0
    if k < M:
        z = logits.view(T, G, M)
        srt = torch.sort(z, dim=-1, descending=True).values
        margin = srt[..., k - 1] - srt[..., k]
        for t0 in range(0, T, 16384):
            t1 = min(T, t0 + 16384)
            scale = (x[t0:t1].float().abs() @ w_r.float().abs().T).view(t1 - t0, G, M) + 1.0
            if b_r is not None:
                scale = scale + b_r.abs().view(1, G, M)
            near += int((margin[t0:t1] <= 2e-5 * scale.max(-1).values).sum())
    return {"per_group_expert_tokens": counts.astype(int).tolist(),
            "max_expert_share": round(float(share.max()), 4), "min_expert_share": round(float(share.min()), 4),
            "near_tie_pairs": near, "pairs": T * G}


def cpu_info() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(cfg, inp, n_rows: int) -> dict:
    """Time the CPU oracle on a bounded sample of the prefill workload:
    routing of the sampled tokens, the attention of every selected head and
    the shared head at those tokens (full causal history each), and their
    slot assembly + W_O. Throughput = the sample's algorithmic FLOP / time."""
    import oracle
    from threadpoolctl import threadpool_info

    rng = np.random.default_rng(7)
    pos = np.sort(rng.choice(cfg.S, size=n_rows, replace=False))
    f64 = synth.to_f64
    x = f64(inp["x"][pos])
    w_r = f64(inp["w_r"])
    q = f64(inp["q"][0:1])
    kk = f64(inp["k"][0:1])
    vv = f64(inp["v"][0:1])
    w_o = f64(inp["w_o"])
    t0 = time.perf_counter()
    z, p, idx, w = oracle.route(x, w_r, cfg.G, cfg.M, cfg.k)
    idx_full = np.zeros((1, cfg.S, cfg.G, cfg.k), np.int64)
    idx_full[0, pos] = idx
    o_r, o_s = oracle.prefill(q, kk, vv, idx_full, cfg.M, positions=pos)
    y = oracle.out_proj(o_r[0], w, o_s[0], w_o)
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(y))
    d, G, k, D, M = cfg.d, cfg.G, cfg.k, cfg.D, cfg.M
    flop = (4 * d * (G * k + 1) * int(np.sum(pos + 1)) + 2 * n_rows * D * G * M
            + 2 * n_rows * (G * k + 2) * d * D)
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} random query positions of the {cfg.name} prefill (all {G * k + 1} "
                      f"selected+shared rows each, full causal history), fp64 NumPy, {dt:.1f} s; "
                      f"BLAS threads={threads}, elementwise ops single-threaded; CPU: {cpu_info()}",
            "seconds": dt}


def prefill_config_line(name: str, steps: int, warmup: int, dev) -> dict:
    """One more prefill workload, timed on its own after the step: the router
    (with lists), the attention and the output projection, each launch
    bracketed by HIP events on the current stream. The attention's roofline is
    its FLOP per launch / mean launch time against the bf16 MFMA peak. A
    sequence of a million tokens (about a second per attention launch) is
    timed over at most two launches after one warmup."""
    cfg = synth.workload(name)
    if cfg.S >= 1 << 20:
        steps, warmup = min(steps, 2), min(warmup, 1)
    inp = synth.make_prefill_inputs(cfg, project=False)
    g = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    B, S, D, N, G, k, d, M, T = cfg.B, cfg.S, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.M, cfg.T
    # Q, K, V prepared on the device in fp32 and rounded to bf16 (input preparation)
    xf = g["x"].float()
    q = (xf @ g["w_q"].float().T).to(torch.bfloat16).view(B, S, N + 1, d).contiguous()
    kk = (xf @ g["w_k"].float().T).to(torch.bfloat16).view(B, S, G, d).permute(0, 2, 1, 3).contiguous()
    vv = (xf @ g["w_v"].float().T).to(torch.bfloat16).view(B, S, G, d).permute(0, 2, 1, 3).contiguous()
    del xf
    dims = gqe.gqe_dims.from_config(cfg)
    r = gqe.route(dims, g["x"], g["w_r"], g["b_r"])
    o_r = torch.empty((B, S, G, k, d), dtype=torch.bfloat16, device=dev)
    o_s = torch.empty((B, S, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    r_ws = torch.empty((max(gqe.gqe_route_workspace_bytes(dims), 16),), dtype=torch.uint8, device=dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    recs = []
    for it in range(warmup + steps):
        e = [ev() for _ in range(4)]
        e[0].record()
        gqe.gqe_route(dims, g["x"], g["w_r"], g["b_r"], None, r["topk_idx"], r["topk_w"], r["list_off"],
                      r["list_tok"], r_ws)
        e[1].record()
        gqe.gqe_attn_prefill(dims, q, kk, vv, r["topk_idx"], o_r, o_s)
        e[2].record()
        gqe.gqe_out_proj(dims, T, o_r.view(T, G, k, d), r["topk_w"], o_s.view(T, d), g["w_o"], y)
        e[3].record()
        if it >= warmup:
            recs.append(e)
    torch.cuda.synchronize()

    def span(i, j):
        return np.array([e[i].elapsed_time(e[j]) for e in recs]) * 1e-3

    fl = prefill_path_flops(cfg)
    t_attn, t_path, t_proj = span(1, 2), span(0, 3), span(2, 3)
    a = fl["attention"] / t_attn.mean()
    pj = 2 * T * (G * k + 2) * d * D
    kern = "prefill_d128_kernel" if d == 128 else "prefill_qp_kernel<%d>" % d
    return {
        "config": {"B": B, "S": S, "D": D, "N": N, "G": G, "M": M, "k": k, "head_dim": d,
                   "skewed_router": cfg.skew},
        "value": round(fl["total"] / t_path.mean() / 1e12, 2), "unit": "TFLOP/s",
        "roofline": {"kernel": f"{kern} (gqe_attn_prefill)", "bound": "mfma", "achieved": round(a / 1e12, 2),
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s", "frac": round(a / PEAK_BF16_FLOPS, 4),
                     "flop_per_launch": fl["attention"],
                     "traffic": (measured_traffic("prefill.hip", "prefill_d128_llama_s8k_pmc.txt")
                                 if name == "llama_s8k_skew" else None)},
        "steps": steps, "warmup": warmup,
        "attention_ms": round(t_attn.mean() * 1e3, 4),
        "attention_min_ms": round(t_attn.min() * 1e3, 4),
        "route_ms": round(span(0, 1).mean() * 1e3, 4),
        "out_proj_ms": round(t_proj.mean() * 1e3, 4),
        "out_proj_frac": round(pj / t_proj.mean() / PEAK_BF16_FLOPS, 4),
        "path_ms": round(t_path.mean() * 1e3, 4),
        "routing": routing_stats(dims, cfg, g["x"], g["w_r"], g["b_r"], r["logits"], r["list_off"]),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_s128k")
    ap.add_argument("--decode-workload", default="decode_kv64k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=3072)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (for counter calibration)")
    ap.add_argument("--extra", default="main_s2k,llama_s8k_skew,long_s1m",
                    help="further prefill workloads timed after the step (comma-separated, '' for none)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this build has no "
              f"multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    gqe.load_library()

    cfg = synth.workload(args.workload)
    dcfg = synth.workload(args.decode_workload)
    print(f"[bench] generating inputs: {cfg.name}, {dcfg.name}", file=sys.stderr, flush=True)
    inp = synth.make_prefill_inputs(cfg)
    dinp = synth.make_decode_inputs(dcfg)
    g = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    dg = {k: (v.to(dev) if v is not None else None) for k, v in dinp.items()}
    dims = gqe.gqe_dims.from_config(cfg)
    ddims = gqe.gqe_dims.from_config(dcfg)
    rdims = gqe.gqe_dims.make(dcfg.B, dcfg.q_len, dcfg.D, dcfg.N, dcfg.G, dcfg.k, dcfg.d, dcfg.dtype)

    # outputs and workspaces, allocated once
    T, G, M, k, d = cfg.T, cfg.G, cfg.M, cfg.k, cfg.d
    r_out = dict(logits=None,
                 topk_idx=torch.empty((T, G, k), dtype=torch.int32, device=dev),
                 topk_w=torch.empty((T, G, k), dtype=torch.float32, device=dev),
                 list_off=torch.empty((cfg.B, G, M + 1), dtype=torch.int32, device=dev),
                 list_tok=torch.empty((cfg.B, G, k * cfg.S), dtype=torch.int32, device=dev))
    r_ws = torch.empty((max(gqe.gqe_route_workspace_bytes(dims), 16),), dtype=torch.uint8, device=dev)
    o_r = torch.empty((cfg.B, cfg.S, G, k, d), dtype=torch.bfloat16, device=dev)
    o_s = torch.empty((cfg.B, cfg.S, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, cfg.D), dtype=torch.bfloat16, device=dev)
    dT = dcfg.T
    d_idx = torch.empty((dT, dcfg.G, dcfg.k), dtype=torch.int32, device=dev)
    d_w = torch.empty((dT, dcfg.G, dcfg.k), dtype=torch.float32, device=dev)
    d_ws = gqe.decode_workspace(ddims, dcfg.q_len, dev)
    d_or = torch.empty((dcfg.B, dcfg.q_len, dcfg.G, dcfg.k, dcfg.d), dtype=torch.bfloat16, device=dev)
    d_os = torch.empty((dcfg.B, dcfg.q_len, dcfg.d), dtype=torch.bfloat16, device=dev)
    d_y = torch.empty((dT, dcfg.D), dtype=torch.bfloat16, device=dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(rec):
        e = [ev() for _ in range(8)]
        e[0].record()
        gqe.gqe_route(dims, g["x"], g["w_r"], g["b_r"], None, r_out["topk_idx"], r_out["topk_w"],
                      r_out["list_off"], r_out["list_tok"], r_ws)
        e[1].record()
        gqe.gqe_attn_prefill(dims, g["q"], g["k"], g["v"], r_out["topk_idx"], o_r, o_s)
        e[2].record()
        gqe.gqe_out_proj(dims, T, o_r.view(T, G, k, d), r_out["topk_w"], o_s.view(T, d), g["w_o"], y)
        e[3].record()
        gqe.gqe_route(rdims, dg["x"], dg["w_r"], dg["b_r"], None, d_idx, d_w, None, None, None)
        e[4].record()
        gqe.gqe_attn_decode(ddims, dcfg.q_len, dg["q"], dg["k"], dg["v"], dg["kv_len"], d_idx,
                            d_or, d_os, d_ws)
        e[5].record()
        gqe.gqe_out_proj(ddims, dT, d_or.view(dT, dcfg.G, dcfg.k, dcfg.d), d_w,
                         d_os.view(dT, dcfg.d), dg["w_o"], d_y)
        e[6].record()
        rec.append(e)

    if args.copy_calibration:
        a = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    warm = []
    for _ in range(args.warmup):
        step(warm)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr,
          flush=True)

    recs = []
    t_begin, t_end = ev(), ev()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_begin.record()
    for _ in range(args.steps):
        step(recs)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t_begin.elapsed_time(t_end)

    def span(i, j):
        return np.array([r[i].elapsed_time(r[j]) for r in recs]) * 1e-3  # seconds

    t_route, t_attn, t_proj = span(0, 1), span(1, 2), span(2, 3)
    t_prefill = span(0, 3)
    t_droute, t_dec, t_dproj = span(3, 4), span(4, 5), span(5, 6)
    t_decode = span(3, 6)

    fl = prefill_path_flops(cfg)
    value = fl["total"] / t_prefill.mean() / 1e12
    attn_tflops = fl["attention"] / t_attn.mean() / 1e12
    kv = decode_kv_bytes(dcfg)
    dec_gbps = kv / t_dec.mean() / 1e9

    # The Q/K/V projections (token-compacted Q) precede the path; they are
    # timed on their own after the steps and reported beside the step, not
    # inside it.
    q_p = torch.zeros((cfg.B, cfg.S, cfg.N + 1, d), dtype=torch.bfloat16, device=dev)
    k_p = torch.empty((cfg.B, G, cfg.S, d), dtype=torch.bfloat16, device=dev)
    v_p = torch.empty_like(k_p)
    x3 = g["x"].view(cfg.B, cfg.S, cfg.D)
    dq_p = torch.empty((dcfg.B, dcfg.q_len, dcfg.N + 1, dcfg.d), dtype=torch.bfloat16, device=dev)
    dx3 = dg["x"].view(dcfg.B, dcfg.q_len, dcfg.D)

    def proj_call():
        gqe.gqe_qkv_proj(dims, x3, g["w_q"], g["w_k"], g["w_v"], r_out["topk_idx"], q_p, k_p, v_p)

    def dproj_call():
        gqe.gqe_qkv_proj_decode(ddims, dcfg.q_len, dx3, dg["w_q"], dg["w_k"], dg["w_v"], d_idx,
                                dg["kv_len"], dq_p, dg["k"], dg["v"])

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        es = [(ev(), ev()) for _ in range(n)]
        for a, b in es:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in es]) * 1e-3

    t_qkv = timed(proj_call, args.steps)
    t_dqkv = timed(dproj_call, args.steps)

    # The whole decode step (routing, projections with the K/V append,
    # attention, output projection) launched call by call, and the same calls
    # captured once in a HIP graph and replayed: a step of small launches,
    # where the graph removes the gaps between them.
    def dstep_calls():
        gqe.gqe_route(rdims, dg["x"], dg["w_r"], dg["b_r"], None, d_idx, d_w, None, None, None)
        gqe.gqe_qkv_proj_decode(ddims, dcfg.q_len, dx3, dg["w_q"], dg["w_k"], dg["w_v"], d_idx,
                                dg["kv_len"], dq_p, dg["k"], dg["v"])
        gqe.gqe_attn_decode(ddims, dcfg.q_len, dq_p, dg["k"], dg["v"], dg["kv_len"], d_idx, d_or, d_os, d_ws)
        gqe.gqe_out_proj(ddims, dT, d_or.view(dT, dcfg.G, dcfg.k, dcfg.d), d_w, d_os.view(dT, dcfg.d),
                         dg["w_o"], d_y)

    t_dstep = timed(dstep_calls, args.steps)

    # The output projection's ablation slot layouts (hard slots alone; hard
    # slots times the selected router probabilities), timed on the step's
    # attention outputs: W_O has G*k*d rows, there is no obar and no shared slot.
    p_sel = torch.empty((T, G, k), dtype=torch.float32, device=dev)
    gqe.gqe_route(dims, g["x"], g["w_r"], g["b_r"], None, r_out["topk_idx"], r_out["topk_w"], None, None, None,
                  topk_p=p_sel)
    w_o_hard = g["w_o"][:G * k * d].contiguous()
    y_abl = torch.empty_like(y)
    t_abl = {}
    for name, code, sw in (("hard", gqe.GQE_SLOTS_HARD, None), ("weighted", gqe.GQE_SLOTS_WEIGHTED, p_sel)):
        t_abl[name] = timed(lambda: gqe.gqe_out_proj_variant(dims, code, T, o_r.view(T, G, k, d), sw, None, w_o_hard,
                                                             y_abl), args.steps)
    abl_flop = 2 * T * G * k * d * cfg.D
    del y_abl, w_o_hard, p_sel
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dstep_calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph):
        dstep_calls()
    torch.cuda.synchronize()
    t_dgraph = timed(dgraph.replay, args.steps)
    del dgraph
    # for comparison: one dense bf16 product (torch -> hipBLASLt) of every
    # query head, K and V, the work the token compaction avoids
    w_all = torch.cat([g["w_q"], g["w_k"], g["w_v"]], 0).contiguous()
    dense_out = torch.empty((T, w_all.shape[0]), dtype=torch.bfloat16, device=dev)

    def dense_call():
        torch.matmul(g["x"], w_all.t(), out=dense_out)

    t_dense = timed(dense_call, args.steps)
    dense_flop = 2 * T * cfg.D * w_all.shape[0]
    del dense_out, w_all
    qkv_flop = projection_flops(T, cfg.D, G, k, d)
    sel = np.unique(d_idx.view(dT, dcfg.G, dcfg.k).cpu().numpy()
                    + dcfg.M * np.arange(dcfg.G)[None, :, None])
    dqkv_bytes = (sel.size + 1 + 2 * dcfg.G) * dcfg.d * dcfg.D * 2  # weights of the heads in use
    qkv = {
        "prefill_ms": round(t_qkv.mean() * 1e3, 4),
        "prefill_tflops": round(qkv_flop / t_qkv.mean() / 1e12, 2),
        "prefill_frac": round(qkv_flop / t_qkv.mean() / PEAK_BF16_FLOPS, 4),
        "prefill_flop": qkv_flop,
        "dense_all_heads_ms": round(t_dense.mean() * 1e3, 4),
        "dense_all_heads_flop": dense_flop,
        "dense_all_heads_tflops": round(dense_flop / t_dense.mean() / 1e12, 2),
        "decode_us": round(t_dqkv.mean() * 1e6, 2),
        "decode_weight_gbps": round(dqkv_bytes / t_dqkv.mean() / 1e9, 1),
        "decode_weight_bytes": int(dqkv_bytes),
    }

    # The same decode against a paged cache: 256-key pages in a seeded random
    # order (gqe_attn_decode_paged), timed after the steps.
    page = 256
    mp = dcfg.S // page
    perm = torch.randperm(dcfg.B * mp, generator=torch.Generator().manual_seed(1)).to(dev)
    kp = torch.empty((dcfg.B * mp, dcfg.G, page, dcfg.d), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    kp[perm] = dg["k"].view(dcfg.B, dcfg.G, mp, page, dcfg.d).permute(0, 2, 1, 3, 4).reshape(kp.shape)
    vp[perm] = dg["v"].view(dcfg.B, dcfg.G, mp, page, dcfg.d).permute(0, 2, 1, 3, 4).reshape(vp.shape)
    bt = perm.to(torch.int32).view(dcfg.B, mp)

    def paged_call():
        gqe.gqe_attn_decode_paged(ddims, dcfg.q_len, dg["q"], kp, vp, bt, page, None, dg["kv_len"], d_idx,
                                  d_or, d_os, d_ws)

    t_paged = timed(paged_call, args.steps)
    del kp, vp
    paged_gbps = kv / t_paged.mean() / 1e9

    # The training backward of the same layer (attention, output projection,
    # router with the balance loss), timed after the steps on seeded output
    # gradients; the training forward supplies the rows' log-sum-exp.
    gen = torch.Generator(device=dev).manual_seed(5)
    lse_r = torch.empty((cfg.B, cfg.S, G, k), dtype=torch.float32, device=dev)
    lse_s = torch.empty((cfg.B, cfg.S), dtype=torch.float32, device=dev)
    gqe.gqe_attn_prefill_train(dims, g["q"], g["k"], g["v"], r_out["topk_idx"], o_r, o_s, lse_r, lse_s)
    do_r = torch.randn(o_r.shape, device=dev, generator=gen).to(torch.bfloat16)
    do_s = torch.randn(o_s.shape, device=dev, generator=gen).to(torch.bfloat16)
    dq_t = torch.zeros_like(g["q"])
    dk_t = torch.empty_like(g["k"])
    dv_t = torch.empty_like(g["v"])
    b_ws = torch.empty((max(gqe.gqe_attn_prefill_bwd_workspace_bytes(dims), 16),), dtype=torch.uint8, device=dev)

    def attn_bwd_call():
        gqe.gqe_attn_prefill_bwd(dims, g["q"], g["k"], g["v"], r_out["topk_idx"], o_r, o_s, lse_r, lse_s,
                                 do_r, do_s, dq_t, dk_t, dv_t, b_ws)

    t_abwd = timed(attn_bwd_call, max(2, args.steps // 2))
    del b_ws
    dy = torch.randn((T, cfg.D), device=dev, generator=gen).to(torch.bfloat16)
    dor_t, dos_t = torch.empty((T, G, k, d), dtype=torch.bfloat16, device=dev), torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    dw_t = torch.empty((T, G, k), dtype=torch.float32, device=dev)
    dwo_t = torch.empty(tuple(g["w_o"].shape), dtype=torch.float32, device=dev)
    o_ws = torch.empty((max(gqe.gqe_out_proj_bwd_workspace_bytes(dims, gqe.GQE_SLOTS_FULL, T), 16),),
                       dtype=torch.uint8, device=dev)

    def oproj_bwd_call():
        gqe.gqe_out_proj_bwd(dims, gqe.GQE_SLOTS_FULL, T, o_r.view(T, G, k, d), r_out["topk_w"], o_s.view(T, d),
                             g["w_o"], dy, dor_t, dw_t, dos_t, dwo_t, o_ws)

    t_obwd = timed(oproj_bwd_call, args.steps)
    del o_ws
    z_t = torch.empty((T, G, M), dtype=torch.float32, device=dev)
    gqe.gqe_route(dims, g["x"], g["w_r"], g["b_r"], z_t, r_out["topk_idx"], r_out["topk_w"], None, None, None)
    dz_t, dx_t = torch.empty_like(z_t), torch.empty_like(g["x"])
    dwr_t = torch.empty((G * M, cfg.D), dtype=torch.float32, device=dev)
    dbr_t = torch.empty((G * M,), dtype=torch.float32, device=dev)
    aux_t = torch.empty((1,), dtype=torch.float32, device=dev)
    rb_ws = torch.empty((max(gqe.gqe_route_bwd_workspace_bytes(dims), 16),), dtype=torch.uint8, device=dev)

    def route_bwd_call():
        gqe.gqe_route_bwd(dims, g["x"], g["w_r"], z_t, r_out["topk_idx"], dw_t, 0.01, dz_t, dx_t, dwr_t, dbr_t,
                          aux_t, rb_ws)

    t_rbwd = timed(route_bwd_call, args.steps)
    del rb_ws
    # five products per (row, visible key) pair, the forward's two plus three
    abwd_flop = fl["attention"] * 5 // 2
    slot_cols = (G * k + 2) * d
    obwd_flop = 2 * 2 * T * slot_cols * cfg.D  # dA = dy W_O^T and dW_O = A^T dy
    rbwd_flop = 2 * 2 * T * G * M * cfg.D      # dW_r = dz^T x and dx = dz W_r
    train_bwd = {
        "attention_ms": round(t_abwd.mean() * 1e3, 4),
        "attention_tflops": round(abwd_flop / t_abwd.mean() / 1e12, 2),
        "attention_frac": round(abwd_flop / t_abwd.mean() / PEAK_BF16_FLOPS, 4),
        "attention_flop": int(abwd_flop),
        "out_proj_ms": round(t_obwd.mean() * 1e3, 4),
        "out_proj_tflops": round(obwd_flop / t_obwd.mean() / 1e12, 2),
        "route_ms": round(t_rbwd.mean() * 1e3, 4),
        "route_tflops": round(rbwd_flop / t_rbwd.mean() / 1e12, 2),
        "balance_loss_coef": 0.01,
    }

    # realised routing of the step's prefill (z_t holds its logits, r_out its lists)
    routing = routing_stats(dims, cfg, g["x"], g["w_r"], g["b_r"], z_t, r_out["list_off"])
    del dz_t, dx_t, z_t
    extra = {}
    for name in [n for n in args.extra.split(",") if n]:
        print(f"[bench] prefill workload {name}", file=sys.stderr, flush=True)
        extra[name] = prefill_config_line(name, args.steps, args.warmup, dev)
        torch.cuda.empty_cache()

    traffic = measured_traffic("prefill.hip", "prefill_long_s128k_pmc.txt")
    dtraffic = measured_traffic("decode.hip", "decode_kv64k_pmc.txt")
    result = {
        "metric": "GQE prefill TFLOP/s & decode KV GB/s at 1 GPU, % of MI355X bf16/HBM peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights; no dataset, random weights)",
        "config": {
            "workload": f"{cfg.name} prefill layer + {dcfg.name} decode step",
            "prefill": {"B": cfg.B, "S": cfg.S, "D": cfg.D, "N": cfg.N, "G": cfg.G, "M": cfg.M,
                        "k": cfg.k, "head_dim": cfg.d, "shared_head": True},
            "decode": {"B": dcfg.B, "q_len": dcfg.q_len, "kv_len": dcfg.kv_len, "D": dcfg.D, "N": dcfg.N,
                       "G": dcfg.G, "M": dcfg.M, "k": dcfg.k, "head_dim": dcfg.d},
        },
        "roofline": {
            "kernel": "prefill_qp_kernel<64> (gqe_attn_prefill)",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_FLOPS / 1e12,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops * 1e12 / PEAK_BF16_FLOPS, 4),
            "traffic": traffic,
        },
        "decode": {
            "value": round(dec_gbps, 1),
            "unit": "GB/s",
            "roofline": {
                "kernel": "decode_split_kernel + decode_combine_kernel (gqe_attn_decode)",
                "bound": "hbm",
                "achieved": round(dec_gbps, 1),
                "peak": PEAK_HBM_BPS / 1e9,
                "unit": "GB/s",
                "frac": round(dec_gbps * 1e9 / PEAK_HBM_BPS, 4),
                "traffic": dtraffic,
            },
            "ms_per_call": round(t_dec.mean() * 1e3, 4),
            "path_ms": round(t_decode.mean() * 1e3, 4),
            "step_with_projections": {"eager_ms": round(t_dstep.mean() * 1e3, 4),
                                      "hip_graph_ms": round(t_dgraph.mean() * 1e3, 4)},
            "paged": {"page_size": page, "order": "shuffled", "value": round(paged_gbps, 1), "unit": "GB/s",
                      "frac": round(paged_gbps * 1e9 / PEAK_HBM_BPS, 4),
                      "ms_per_call": round(t_paged.mean() * 1e3, 4)},
        },
        "breakdown_ms": {
            "prefill_route": round(t_route.mean() * 1e3, 4),
            "prefill_attention": round(t_attn.mean() * 1e3, 4),
            "prefill_out_proj": round(t_proj.mean() * 1e3, 4),
            "decode_route": round(t_droute.mean() * 1e3, 4),
            "decode_attention": round(t_dec.mean() * 1e3, 4),
            "decode_out_proj": round(t_dproj.mean() * 1e3, 4),
            "attention_min_ms": round(t_attn.min() * 1e3, 4),
            "attention_max_ms": round(t_attn.max() * 1e3, 4),
        },
        "routing": routing,
        "prefill_workloads": extra,
        "qkv_proj": qkv,
        "ablation_out_proj": {
            name: {"ms": round(t_abl[name].mean() * 1e3, 4), "flop": abl_flop,
                   "tflops": round(abl_flop / t_abl[name].mean() / 1e12, 2),
                   "frac": round(abl_flop / t_abl[name].mean() / PEAK_BF16_FLOPS, 4)}
            for name in ("hard", "weighted")},
        "train_bwd": train_bwd,
        "flop_per_step": fl,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu:
        print(f"[bench] timing the CPU oracle on {args.cpu_rows} sampled rows", file=sys.stderr, flush=True)
        cb = cpu_baseline(cfg, inp, args.cpu_rows)
        result["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in cb.items()}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
