"""Seeded synthetic workloads for the GQE attention layer.

This module only *generates inputs*. It holds none of the layer's arithmetic
(routing, attention, slot assembly, output projection); both the CPU oracle
and the GPU path receive the tensors made here.

Recipe (one fixed draw order per workload, ``numpy.random.default_rng(seed)``,
float32 ``standard_normal``):

* prefill: x [B,S,D] ~ N(0,1); then W_Q [(N+1)*d, D], W_K [G*d, D],
  W_V [G*d, D], W_r [G*M, D], W_O [(G*k+2)*d, D_out=D] each ~ N(0,1) * 0.02
  (0.02 is the standard deviation).
* decode: x [B,q_len,D] ~ N(0,1); then W_Q, W_r, W_O as above. The KV cache
  K,V [B,G,S_max,d] ~ N(0,1) is drawn per (b, g) block from
  ``default_rng([seed, b, g, t])`` with t=0 for K and t=1 for V, so blocks can
  be drawn in parallel threads. The decode layer's W_K and W_V (used only
  to project and append the new tokens' keys and values) come from
  ``default_rng([seed, 303])``, so the draws above are unchanged.
* bf16 workloads round x and every weight to bfloat16 (round to nearest even).
  Q, K and V are the fp32 products x @ W^T of those rounded values, then
  rounded to bfloat16. The projections are input preparation, not part of the
  layer measured here.
* The skewed-router workload adds a router bias of ln 3 to expert
  m* = g mod M of every group g: 3:1 odds for that expert against an equally
  scored rival.
* attention-only (a sequence too long to project on the host): q
  [B,S,N+1,d], then k and v [B,G,S,d], drawn directly from
  ``default_rng([seed, 404])`` as N(0,1) * 0.02 * sqrt(D), the distribution of
  an entry of x @ W^T above, in chunks of 65536 positions (same draw order),
  rounded to the workload dtype.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np
import torch

__all__ = [
    "GQEConfig", "WORKLOADS", "workload", "make_prefill_inputs",
    "make_attention_inputs", "make_decode_inputs", "to_f64", "round_bf16",
]


@dataclasses.dataclass(frozen=True)
class GQEConfig:
    """Shape of one GQE layer invocation.

    N routed query heads in G groups (M = N/G experts per group), top-k per
    group, one extra always-on shared query head (column block N of Q), head
    dimension d, model width D.
    """

    name: str
    B: int
    S: int
    D: int
    N: int
    G: int
    k: int
    d: int
    dtype: str = "bf16"          # "bf16" or "f32"
    seed: int = 0
    skew: bool = False           # bias ln 3 on expert g mod M of each group
    mode: str = "prefill"        # "prefill" or "decode"
    q_len: int = 1               # decode only: new tokens per sequence
    kv_len: Optional[int] = None  # decode only: valid cache length (default S)

    @property
    def M(self) -> int:
        return self.N // self.G

    @property
    def T(self) -> int:
        return self.B * (self.q_len if self.mode == "decode" else self.S)

    @property
    def slot_width(self) -> int:
        """Width of the assembled slot vector: G*k hard slots, weighted sum, shared."""
        return (self.G * self.k + 2) * self.d

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "GQEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads the layer is measured and checked on.
WORKLOADS = {
    # tiny fp32 layer: the small case the oracle finishes in well under a second
    "tiny_f32": GQEConfig("tiny_f32", B=1, S=128, D=256, N=4, G=2, k=1, d=32, dtype="f32"),
    # the pages' main layer: 16 query heads, 8 KV heads, 2 experts per group, top-1
    "main_s2k": GQEConfig("main_s2k", B=8, S=2048, D=1024, N=16, G=8, k=1, d=64),
    # long-context prefill, same layer
    "long_s128k": GQEConfig("long_s128k", B=1, S=131072, D=1024, N=16, G=8, k=1, d=64),
    # the long-context layer at 1,048,576 tokens (the far end of the pages' 4k-1024k range)
    "long_s1m": GQEConfig("long_s1m", B=1, S=1048576, D=1024, N=16, G=8, k=1, d=64),
    # Llama-shaped layer with a skewed router
    "llama_s8k_skew": GQEConfig("llama_s8k_skew", B=2, S=8192, D=4096, N=32, G=8, k=2,
                                d=128, skew=True),
    # decode: 16 sequences x 1 new token against 65536 cached keys each
    "decode_kv64k": GQEConfig("decode_kv64k", B=16, S=65536, D=4096, N=32, G=8, k=2,
                              d=128, mode="decode", q_len=1, kv_len=65536),
}


def workload(name: str, **overrides) -> GQEConfig:
    return WORKLOADS[name].replace(**overrides) if overrides else WORKLOADS[name]


def round_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 ndarray -> bfloat16 tensor, round to nearest even."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def to_f64(t) -> np.ndarray:
    """Exact upcast of a bf16/fp32 tensor (any device) or ndarray to float64 numpy."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def _store(a: np.ndarray, cfg: GQEConfig) -> torch.Tensor:
    if cfg.dtype == "bf16":
        return round_bf16(a)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def _router_bias(cfg: GQEConfig) -> Optional[torch.Tensor]:
    if not cfg.skew:
        return None
    b = np.zeros((cfg.G, cfg.M), dtype=np.float32)
    for g in range(cfg.G):
        b[g, g % cfg.M] = math.log(3.0)
    return torch.from_numpy(b.reshape(-1))


def _proj(x: torch.Tensor, w: torch.Tensor, cfg: GQEConfig) -> torch.Tensor:
    """fp32 product x @ w^T of stored values, stored back in the workload dtype."""
    y = x.float() @ w.float().T
    return y.to(cfg.torch_dtype)


def make_prefill_inputs(cfg: GQEConfig, project: bool = True) -> dict:
    """CPU tensors for one prefill invocation (see the module docstring).
    With ``project`` False the prepared q, k, v are left out (the draws are
    the same)."""
    assert cfg.mode == "prefill"
    B, S, D, N, G, k, d, M = cfg.B, cfg.S, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.M
    rng = np.random.default_rng(cfg.seed)
    x = _store(rng.standard_normal((B * S, D), dtype=np.float32), cfg)
    w_q = _store(rng.standard_normal(((N + 1) * d, D), dtype=np.float32) * np.float32(0.02), cfg)
    w_k = _store(rng.standard_normal((G * d, D), dtype=np.float32) * np.float32(0.02), cfg)
    w_v = _store(rng.standard_normal((G * d, D), dtype=np.float32) * np.float32(0.02), cfg)
    w_r = _store(rng.standard_normal((G * M, D), dtype=np.float32) * np.float32(0.02), cfg)
    w_o = _store(rng.standard_normal(((G * k + 2) * d, D), dtype=np.float32) * np.float32(0.02), cfg)
    q = kk = vv = None
    if project:
        q = _proj(x, w_q, cfg).reshape(B, S, N + 1, d).contiguous()
        kk = _proj(x, w_k, cfg).reshape(B, S, G, d).permute(0, 2, 1, 3).contiguous()
        vv = _proj(x, w_v, cfg).reshape(B, S, G, d).permute(0, 2, 1, 3).contiguous()
    return dict(x=x, w_r=w_r, b_r=_router_bias(cfg), q=q, k=kk, v=vv, w_o=w_o, w_q=w_q, w_k=w_k, w_v=w_v)


def make_attention_inputs(cfg: GQEConfig) -> dict:
    """CPU tensors q, k, v for the attention alone (see the module docstring),
    drawn without the projection so that sequences of a million tokens stay
    cheap to make."""
    B, S, N, G, d = cfg.B, cfg.S, cfg.N, cfg.G, cfg.d
    rng = np.random.default_rng([cfg.seed, 404])
    sd = np.float32(0.02 * math.sqrt(cfg.D))
    q = torch.empty((B, S, N + 1, d), dtype=cfg.torch_dtype)
    k = torch.empty((B, G, S, d), dtype=cfg.torch_dtype)
    v = torch.empty((B, G, S, d), dtype=cfg.torch_dtype)
    C = 65536
    for b in range(B):
        for s0 in range(0, S, C):
            n = min(C, S - s0)
            q[b, s0:s0 + n] = _store(rng.standard_normal((n, N + 1, d), dtype=np.float32) * sd, cfg)
    for t in (k, v):
        for b in range(B):
            for g in range(G):
                for s0 in range(0, S, C):
                    n = min(C, S - s0)
                    t[b, g, s0:s0 + n] = _store(rng.standard_normal((n, d), dtype=np.float32) * sd, cfg)
    return dict(q=q, k=k, v=v)


def _cache_block(seed: int, b: int, g: int, t: int, S: int, d: int, bf16: bool):
    a = np.random.default_rng([seed, b, g, t]).standard_normal((S, d), dtype=np.float32)
    return round_bf16(a) if bf16 else torch.from_numpy(a)


def make_decode_inputs(cfg: GQEConfig, threads: Optional[int] = None) -> dict:
    """CPU tensors for one decode invocation (see the module docstring)."""
    assert cfg.mode == "decode"
    B, S, D, N, G, k, d, M, L = cfg.B, cfg.S, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.M, cfg.q_len
    rng = np.random.default_rng(cfg.seed)
    x = _store(rng.standard_normal((B * L, D), dtype=np.float32), cfg)
    w_q = _store(rng.standard_normal(((N + 1) * d, D), dtype=np.float32) * np.float32(0.02), cfg)
    w_r = _store(rng.standard_normal((G * M, D), dtype=np.float32) * np.float32(0.02), cfg)
    w_o = _store(rng.standard_normal(((G * k + 2) * d, D), dtype=np.float32) * np.float32(0.02), cfg)
    q = _proj(x, w_q, cfg).reshape(B, L, N + 1, d).contiguous()
    kc = torch.empty((B, G, S, d), dtype=cfg.torch_dtype)
    vc = torch.empty((B, G, S, d), dtype=cfg.torch_dtype)
    jobs = [(b, g, t) for b in range(B) for g in range(G) for t in (0, 1)]
    bf16 = cfg.dtype == "bf16"

    def fill(job):
        b, g, t = job
        (kc if t == 0 else vc)[b, g].copy_(_cache_block(cfg.seed, b, g, t, S, d, bf16))

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    with _cf.ThreadPoolExecutor(nthr) as ex:
        list(ex.map(fill, jobs))
    kv_len = cfg.kv_len if cfg.kv_len is not None else S
    kvl = torch.full((B,), kv_len, dtype=torch.int32)
    rng_kv = np.random.default_rng([cfg.seed, 303])
    w_k = _store(rng_kv.standard_normal((G * d, D), dtype=np.float32) * np.float32(0.02), cfg)
    w_v = _store(rng_kv.standard_normal((G * d, D), dtype=np.float32) * np.float32(0.02), cfg)
    return dict(x=x, w_r=w_r, b_r=_router_bias(cfg), q=q, k=kc, v=vc, kv_len=kvl, w_o=w_o, w_q=w_q,
                w_k=w_k, w_v=w_v)


def random_selection(B: int, S: int, G: int, M: int, k: int, seed: int,
                     skew: bool = False) -> torch.Tensor:
    """A seeded random choice of k distinct experts per (token, group), stored
    ascending, as int32 [B*S, G, k]. With ``skew`` the first pick is expert
    g mod M with probability 3/(M+2) (3:1 against each other expert) and the
    remaining k-1 are uniform over the rest. Used to drive the attention and
    projection kernels independently of the router."""
    rng = np.random.default_rng([seed, 101])
    T = B * S
    perm = rng.permuted(np.broadcast_to(np.arange(M), (T, G, M)).copy(), axis=-1)
    if skew and M > 1:
        fav = np.arange(G) % M
        prob = np.ones((G, M))
        prob[np.arange(G), fav] = 3.0
        prob /= prob.sum(-1, keepdims=True)
        u = rng.random((T, G, 1))
        first = (u > np.cumsum(prob, -1)[None]).sum(-1)  # categorical draw per (t, g)
        # move `first` to the front of the permutation
        pos = np.argmax(perm == first[..., None], axis=-1)
        perm[np.arange(T)[:, None], np.arange(G)[None, :], pos] = perm[..., 0]
        perm[..., 0] = first
    sel = np.sort(perm[..., :k], axis=-1).astype(np.int32)
    return torch.from_numpy(np.ascontiguousarray(sel))


def make_slot_inputs(T: int, G: int, k: int, d: int, D: int, dtype: str, seed: int) -> dict:
    """Seeded stand-ins for attention outputs and routing weights, to drive the
    output projection on its own: o_routed [T,G,k,d] and o_shared [T,d] ~ N(0,1)/2,
    weights w [T,G,k] drawn from a flat Dirichlet (positive, summing to 1 per
    (t, g)), W_O [(G*k+2)*d, D] ~ N(0,1)*0.02."""
    rng = np.random.default_rng([seed, 202])
    cast = round_bf16 if dtype == "bf16" else (lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)))
    o_r = cast(rng.standard_normal((T, G, k, d), dtype=np.float32) * np.float32(0.5))
    o_s = cast(rng.standard_normal((T, d), dtype=np.float32) * np.float32(0.5))
    w = torch.from_numpy(rng.dirichlet(np.ones(k), size=(T, G)).astype(np.float32))
    w_o = cast(rng.standard_normal(((G * k + 2) * d, D), dtype=np.float32) * np.float32(0.02))
    return dict(o_r=o_r, o_s=o_s, w=w, w_o=w_o)
