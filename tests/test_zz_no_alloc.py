"""The allocation-free decode (gqe_attn_decode_noalloc) through the C ABI.

Its kernels and split geometry are those of gqe_attn_decode; only the split
partials move from the caller's workspace to the library's static device
scratch. So its outputs must equal gqe_attn_decode's bit for bit, on two calls
in a row, the second smaller (the scratch keeps the first call's partials),
and both must match the CPU oracle within the bf16 bound.
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


def _case(B, q_len, Smax, H, G, k, d, kv_len, seed):
    rng = np.random.default_rng(seed)
    bf = torch.bfloat16
    q = torch.from_numpy(rng.standard_normal((B, q_len, H + 1, d), dtype=np.float32)).to(bf)
    K = torch.from_numpy(rng.standard_normal((B, G, Smax, d), dtype=np.float32)).to(bf)
    V = torch.from_numpy((rng.standard_normal((B, G, Smax, d)) + 0.5 * np.arange(G)[None, :, None, None])
                         .astype(np.float32)).to(bf)
    idx = synth.random_selection(B, q_len, G, H // G, k, seed)
    dims = gqe.gqe_dims.make(B, Smax, 64, H, G, k, d, "bf16")
    return dims, q, K, V, np.asarray(kv_len, dtype=np.int32), idx


def _run_both(dims, q_len, q, K, V, kv_len, idx):
    g = [t.to(DEV) for t in (q, K, V, torch.from_numpy(kv_len), idx)]
    a_r, a_s = gqe.decode(dims, q_len, *g)
    b_r = torch.full_like(a_r, float("nan"))
    b_s = torch.full_like(a_s, float("nan"))
    gqe.gqe_attn_decode_noalloc(dims, q_len, *g, b_r, b_s)
    torch.cuda.synchronize()
    return a_r, a_s, b_r, b_s


def test_decode_noalloc_equals_decode_two_calls():
    # first call: 8 sequences x 8 heads x 32768 keys, d = 128, k = 2 (3.2 MB of partials)
    first = _case(8, 1, 32768, 32, 8, 2, 128, [32768, 1, 20000, 4097, 32767, 2, 16384, 9999], 1)
    # second call, smaller: 3 sequences x 2 heads x 1000 keys, d = 64, two new tokens
    second = _case(3, 2, 1000, 8, 2, 2, 64, [1000, 2, 513], 2)
    for n, (dims, q, K, V, kv_len, idx) in enumerate((first, second)):
        q_len = q.shape[1]
        need = gqe.gqe_decode_workspace_bytes(dims, q_len)
        assert 0 < need <= gqe.gqe_decode_scratch_bytes()
        print(f"call {n}: B={dims.B} q_len={q_len} S_max={dims.S} G={dims.G} d={dims.d}: {need} bytes of partials",
              flush=True)
        a_r, a_s, b_r, b_s = _run_both(dims, q_len, q, K, V, kv_len, idx)
        assert torch.equal(a_r, b_r) and torch.equal(a_s, b_s), f"call {n}: differs from gqe_attn_decode"
        M = dims.N // dims.G
        ref_r, ref_s = oracle.decode(f64(q), f64(K), f64(V), kv_len, idx.numpy().reshape(dims.B, q_len, dims.G,
                                                                                          dims.k), M)
        for got, ref, what in ((b_r, ref_r, "O_routed"), (b_s, ref_s, "O_shared")):
            err = float(np.max(np.abs(f64(got) - ref)))
            print(f"call {n} {what}: max|err|={err:.3e}", flush=True)
            assert err <= 2e-2, f"call {n} {what}: {err:.3e}"


def test_decode_noalloc_rejects_oversized_call():
    """A call whose partials exceed the scratch fails with GQE_ERR_SCRATCH
    and leaves its outputs untouched."""
    B, q_len, Smax, H, G, k, d = 512, 3, 1024, 32, 8, 4, 128
    dims = gqe.gqe_dims.make(B, Smax, 64, H, G, k, d, "bf16")
    assert gqe.gqe_decode_workspace_bytes(dims, q_len) > gqe.gqe_decode_scratch_bytes()
    q = torch.zeros((B, q_len, H + 1, d), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((B, G, Smax, d), dtype=torch.bfloat16, device=DEV)
    kv_len = torch.full((B,), Smax, dtype=torch.int32, device=DEV)
    idx = torch.zeros((B * q_len, G, k), dtype=torch.int32, device=DEV)
    o_r = torch.full((B, q_len, G, k, d), 7.0, dtype=torch.bfloat16, device=DEV)
    o_s = torch.full((B, q_len, d), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gqe.GQEError) as e:
        gqe.gqe_attn_decode_noalloc(dims, q_len, q, kc, kc, kv_len, idx, o_r, o_s)
    assert e.value.status == gqe.GQE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o_r == 7.0).all()) and bool((o_s == 7.0).all())
