"""Paged and left-padded decode (gqe_attn_decode_paged) through the C ABI.

Parity with the CPU oracle on the contiguous cache the pages hold (pages in
a random order, unused pages filled with large values so that a wrong page
shows); with an identity page table and no padding the result must equal
gqe_attn_decode bit for bit (same arithmetic, other addressing), which is
also the check at the decode workload's full size.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_query_gqa_amd as gqe
import synth
from test_gpu_parity import DEV, assert_close, f64

pytestmark = pytest.mark.gpu


def _paged(K, V, page, rng, extra=3):
    """Scatter contiguous caches [B, G, S, d] into a shuffled page pool."""
    B, G, S, d = K.shape
    mp = S // page
    n_pages = B * mp + extra
    order = rng.permutation(n_pages)[:B * mp].reshape(B, mp)
    kp = torch.full((n_pages, G, page, d), 1000.0, dtype=K.dtype)
    vp = torch.full((n_pages, G, page, d), -1000.0, dtype=V.dtype)
    for b in range(B):
        for j in range(mp):
            kp[order[b, j]] = K[b, :, j * page:(j + 1) * page]
            vp[order[b, j]] = V[b, :, j * page:(j + 1) * page]
    return kp, vp, torch.from_numpy(order.astype(np.int32))


CASES = [
    # B, q_len, S_max, page, kv_len, kv_start (or None), H, G, k, d, dtype
    (3, 1, 1024, 64, [1, 700, 1024], [0, 100, 7], 8, 2, 1, 64, "bf16"),
    (2, 2, 2048, 256, [2048, 1500], [1000, 0], 32, 8, 2, 128, "bf16"),
    (4, 3, 512, 128, [3, 64, 200, 512], None, 8, 4, 1, 32, "bf16"),
    (2, 1, 4096, 1024, [4096, 1025], [4000, 0], 16, 8, 1, 64, "bf16"),
    (2, 2, 512, 64, [300, 512], [5, 0], 8, 2, 2, 64, "f32"),
    (2, 1, 256, 64, [256, 70], [0, 69], 4, 1, 2, 128, "f32"),
]


@pytest.mark.parametrize("B,L,Smax,page,kvl,kvs,H,G,k,d,dtype", CASES)
def test_decode_paged_matches_oracle(B, L, Smax, page, kvl, kvs, H, G, k, d, dtype):
    M = H // G
    rng = np.random.default_rng(B * 1000 + Smax + page)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, L, H + 1, d), dtype=np.float32)).to(tdt)
    K = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(tdt)
    V = torch.from_numpy((rng.standard_normal((B, G, Smax, d)) + 0.5 * np.arange(G)[None, :, None, None])
                         .astype(np.float32)).to(tdt)
    kp, vp, bt = _paged(K, V, page, rng)
    kv_len = np.array(kvl, dtype=np.int32)
    kv_start = None if kvs is None else np.array(kvs, dtype=np.int32)
    idx = synth.random_selection(B, L, G, M, k, 4)
    dims = gqe.gqe_dims.make(B, Smax, 64, H, G, k, d, dtype)
    print(f"case B={B} q_len={L} Smax={Smax} page={page} d={d} {dtype}", flush=True)
    o_r, o_s = gqe.decode_paged(dims, L, q.to(DEV), kp.to(DEV), vp.to(DEV), bt.to(DEV), page,
                                torch.from_numpy(kv_len).to(DEV), idx.to(DEV),
                                kv_start=None if kv_start is None else torch.from_numpy(kv_start).to(DEV))
    torch.cuda.synchronize()
    ref_r, ref_s = oracle.decode(f64(q), f64(K), f64(V), kv_len, idx.numpy().reshape(B, L, G, k), M,
                                 kv_start=kv_start)
    assert_close(o_r, ref_r, dtype, "paged O_routed")
    assert_close(o_s, ref_s, dtype, "paged O_shared")


@pytest.mark.parametrize("d,page", [(64, 64), (128, 256), (32, 128)])
def test_decode_paged_identity_equals_contiguous(d, page):
    B, L, Smax, H, G, k = 3, 2, 2048, 16, 8, 2
    M = H // G
    rng = np.random.default_rng(d + page)
    q = torch.from_numpy(rng.standard_normal((B, L, H + 1, d), dtype=np.float32)).to(torch.bfloat16).to(DEV)
    K = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(torch.bfloat16).to(DEV)
    V = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(torch.bfloat16).to(DEV)
    kv_len = torch.tensor([2048, 999, 2], dtype=torch.int32, device=DEV)
    idx = synth.random_selection(B, L, G, M, k, 8).to(DEV)
    dims = gqe.gqe_dims.make(B, Smax, 64, H, G, k, d, "bf16")
    mp = Smax // page
    # identity paging: page b*mp + j holds keys j*page.. of sequence b
    kp = K.view(B, G, mp, page, d).permute(0, 2, 1, 3, 4).contiguous().view(B * mp, G, page, d)
    vp = V.view(B, G, mp, page, d).permute(0, 2, 1, 3, 4).contiguous().view(B * mp, G, page, d)
    bt = torch.arange(B * mp, dtype=torch.int32, device=DEV).view(B, mp)
    a_r, a_s = gqe.decode(dims, L, q, K, V, kv_len, idx)
    b_r, b_s = gqe.decode_paged(dims, L, q, kp, vp, bt, page, kv_len, idx)
    torch.cuda.synchronize()
    assert torch.equal(a_r, b_r) and torch.equal(a_s, b_s)


def test_decode_paged_full_size_shuffled_pages():
    """The decode workload (16 x 65536 keys, d = 128) in 256-key pages in a
    random order gives the contiguous path's result bit for bit."""
    cfg = synth.workload("decode_kv64k")
    B, L, S, H, G, k, d, M = cfg.B, cfg.q_len, cfg.S, cfg.N, cfg.G, cfg.k, cfg.d, cfg.M
    page = 256
    gen = torch.Generator(device=DEV).manual_seed(0)
    K = torch.randn((B, G, S, d), generator=gen, device=DEV).to(torch.bfloat16)
    V = torch.randn((B, G, S, d), generator=gen, device=DEV).to(torch.bfloat16)
    q = torch.randn((B, L, H + 1, d), generator=gen, device=DEV).to(torch.bfloat16)
    kv_len = torch.full((B,), S, dtype=torch.int32, device=DEV)
    idx = synth.random_selection(B, L, G, M, k, 0).to(DEV)
    dims = gqe.gqe_dims.from_config(cfg)
    a_r, a_s = gqe.decode(dims, L, q, K, V, kv_len, idx)
    mp = S // page
    perm = torch.randperm(B * mp, generator=torch.Generator().manual_seed(1)).to(DEV)
    kp = torch.empty((B * mp, G, page, d), dtype=torch.bfloat16, device=DEV)
    vp = torch.empty_like(kp)
    kp[perm] = K.view(B, G, mp, page, d).permute(0, 2, 1, 3, 4).reshape(B * mp, G, page, d)
    vp[perm] = V.view(B, G, mp, page, d).permute(0, 2, 1, 3, 4).reshape(B * mp, G, page, d)
    del K, V
    bt = perm.to(torch.int32).view(B, mp)
    b_r, b_s = gqe.decode_paged(dims, L, q, kp, vp, bt, page, kv_len, idx)
    torch.cuda.synchronize()
    assert torch.equal(a_r, b_r) and torch.equal(a_s, b_s)
