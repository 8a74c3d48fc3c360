"""C ABI checks that need no GPU: the library loads, exports every function
include/gqe.h declares, and rejects bad arguments before enqueuing anything.

Fake device pointers are plain aligned (or deliberately misaligned) integers;
every call here fails validation (or is an empty no-op), so nothing reaches
the HIP runtime.
"""
import ctypes
import os
import re

import pytest

import sparse_query_gqa_amd as gqe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqe.h")

A = 0x100000   # an aligned fake device address
MIS = A + 8    # misaligned by 8 bytes


def _lib():
    if not os.path.exists(gqe.LIB_PATH):
        pytest.skip("libgqe.so not built (run __graft_entry__.build())")
    return gqe.load_library()


def _dims(**kw):
    base = dict(B=2, S=100, D=64, N=8, G=2, k=2, d=64, dtype=gqe.GQE_BF16)
    base.update(kw)
    return gqe.gqe_dims(**base)


def P(v=A):
    return ctypes.c_void_p(v)


def test_header_symbols_exported():
    lib = _lib()
    src = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(gqe_[a-z_0-9]+)\s*\(", src, re.M))
    assert declared == set(gqe.EXPORTED), f"header declares {sorted(declared)}"
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings_and_version():
    lib = _lib()
    for st in (0, -1, -2, -3, -4, -5, -6):
        s = lib.gqe_status_string(st).decode()
        assert s.startswith("GQE_")
    assert lib.gqe_status_string(7).decode() == "unknown gqe status"
    assert lib.gqe_version() == 10000


def route(lib, dims, x=A, w=A, b=None, logits=A, idx=A, wt=A, off=None, tok=None, ws=None, nws=0, pr=None):
    return lib.gqe_route(ctypes.byref(dims), P(x), P(w), None if b is None else P(b),
                         None if logits is None else P(logits), None if idx is None else P(idx),
                         None if wt is None else P(wt), None if pr is None else P(pr),
                         None if off is None else P(off), None if tok is None else P(tok),
                         None if ws is None else P(ws), nws, None)


def test_route_validation():
    lib = _lib()
    assert route(lib, _dims(N=8, G=3)) == gqe.GQE_ERR_UNSUPPORTED     # G does not divide N
    assert route(lib, _dims(k=5)) == gqe.GQE_ERR_UNSUPPORTED          # k > M
    assert route(lib, _dims(k=0)) == gqe.GQE_ERR_INVALID_ARG
    assert route(lib, _dims(d=48)) == gqe.GQE_ERR_UNSUPPORTED
    assert route(lib, _dims(D=60)) == gqe.GQE_ERR_UNSUPPORTED         # D % 8
    assert route(lib, _dims(dtype=7)) == gqe.GQE_ERR_UNSUPPORTED
    assert route(lib, _dims(N=66, G=2, k=1)) == gqe.GQE_ERR_UNSUPPORTED  # M > 32
    assert route(lib, _dims(N=288, G=9, k=1)) == gqe.GQE_ERR_UNSUPPORTED  # G*M > 256
    assert route(lib, _dims(B=-1)) == gqe.GQE_ERR_INVALID_ARG
    assert route(lib, _dims(), x=0) == gqe.GQE_ERR_INVALID_ARG
    assert route(lib, _dims(), idx=None) == gqe.GQE_ERR_INVALID_ARG
    assert route(lib, _dims(), x=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert route(lib, _dims(), logits=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert route(lib, _dims(), pr=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert route(lib, _dims(B=0), pr=A) == gqe.GQE_OK
    assert route(lib, _dims(), off=A) == gqe.GQE_ERR_INVALID_ARG     # off without tok
    need = lib.gqe_route_workspace_bytes(ctypes.byref(_dims()))
    assert need == 2 * 2 * 4 * 2 * 4  # B*G*M*ceil(S/64) int32
    assert route(lib, _dims(), off=A, tok=A) == gqe.GQE_ERR_WORKSPACE
    assert route(lib, _dims(), off=A, tok=A, ws=A, nws=need - 1) == gqe.GQE_ERR_WORKSPACE
    assert route(lib, _dims(), off=A, tok=A, ws=MIS, nws=need) == gqe.GQE_ERR_ALIGNMENT
    # empty calls succeed without touching the device
    assert route(lib, _dims(B=0)) == gqe.GQE_OK
    assert route(lib, _dims(S=0), off=A, tok=A) == gqe.GQE_OK


def test_prefill_validation():
    lib = _lib()

    def call(dims, q=A, k=A, v=A, idx=A, o_r=A, o_s=A):
        return lib.gqe_attn_prefill(ctypes.byref(dims), P(q), P(k), P(v), P(idx), P(o_r), P(o_s), None)

    assert call(_dims(N=8, G=3)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(d=256)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(), q=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), o_s=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), v=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(B=0)) == gqe.GQE_OK
    assert call(_dims(S=0)) == gqe.GQE_OK
    assert lib.gqe_attn_prefill(None, P(), P(), P(), P(), P(), P(), None) == gqe.GQE_ERR_INVALID_ARG
    # one head's keys (S*d*2 bytes) must fit a 32-bit buffer size
    assert call(_dims(B=1, S=(1 << 24), d=128)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(B=0, S=(1 << 24) - 1, d=128)) == gqe.GQE_OK


def test_decode_validation():
    lib = _lib()

    def call(dims, L=1, ws=A, nws=1 << 30, kv=A, q=A):
        return lib.gqe_attn_decode(ctypes.byref(dims), L, P(q), P(A), P(A), P(kv), P(A), P(A), P(A),
                                   None if ws is None else P(ws), nws, None)

    d = _dims(S=65536, N=32, G=8, k=2, d=128)
    need = lib.gqe_decode_workspace_bytes(ctypes.byref(d), 1)
    assert need > 0
    assert call(d, ws=None) == gqe.GQE_ERR_WORKSPACE
    assert call(d, nws=need - 1) == gqe.GQE_ERR_WORKSPACE
    assert call(d, ws=MIS, nws=need) == gqe.GQE_ERR_ALIGNMENT
    assert call(d, L=-1) == gqe.GQE_ERR_INVALID_ARG
    assert call(d, kv=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(d, q=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(S=4), L=5) == gqe.GQE_ERR_INVALID_ARG          # q_len > S_max
    assert call(_dims(S=100, k=2), L=6) == gqe.GQE_ERR_UNSUPPORTED   # (k+1)*q_len > 16
    assert call(_dims(N=8, G=3)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(B=0)) == gqe.GQE_OK
    assert call(d, L=0) == gqe.GQE_OK


def test_decode_noalloc_validation():
    """The allocation-free decode checks what gqe_attn_decode checks, and
    rejects a call whose split partials exceed its static scratch before
    touching the device."""
    lib = _lib()
    assert lib.gqe_decode_scratch_bytes() == 16 << 20

    def call(dims, L=1, kv=A, q=A):
        return lib.gqe_attn_decode_noalloc(ctypes.byref(dims), L, P(q), P(A), P(A), P(kv), P(A), P(A), P(A), None)

    d = _dims(S=65536, N=32, G=8, k=2, d=128)
    assert lib.gqe_decode_workspace_bytes(ctypes.byref(d), 1) <= 16 << 20
    assert call(d, L=-1) == gqe.GQE_ERR_INVALID_ARG
    assert call(d, kv=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(d, q=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(S=4), L=5) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(S=100, k=2), L=6) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(N=8, G=3)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(B=0)) == gqe.GQE_OK
    assert call(d, L=0) == gqe.GQE_OK
    # 512 x 8 heads, one split each, 15 rows of d = 128: 4096*15*(128+2)*4 bytes > 16 MiB
    big = _dims(B=512, S=1024, N=32, G=8, k=4, d=128)
    assert lib.gqe_decode_workspace_bytes(ctypes.byref(big), 3) == 4096 * 15 * 130 * 4
    assert call(big, L=3) == gqe.GQE_ERR_SCRATCH


def test_out_proj_validation():
    lib = _lib()

    def call(dims, T=10, y=A, w=A):
        return lib.gqe_out_proj(ctypes.byref(dims), T, P(A), P(A), P(A), P(w), P(y), None)

    assert call(_dims(), T=-1) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), y=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), w=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(D=12)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(N=8, G=3)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(), T=0) == gqe.GQE_OK
    # a 256-token output tile is addressed through 32-bit byte offsets
    assert call(_dims(D=1 << 23), T=0) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(D=(1 << 23) - 8), T=0) == gqe.GQE_OK


def test_out_proj_variant_validation():
    lib = _lib()

    def call(dims, mode, T=10, y=A, sw=A, os_=A):
        return lib.gqe_out_proj_variant(ctypes.byref(dims), mode, T, P(A), None if sw is None else P(sw),
                                        None if os_ is None else P(os_), P(A), P(y), None)

    assert call(_dims(), 3) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(), -1) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(), gqe.GQE_SLOTS_HARD, y=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_WEIGHTED, T=-1) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_WEIGHTED, y=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(), gqe.GQE_SLOTS_HARD, T=0) == gqe.GQE_OK
    # the ablation layouts read no shared output; the hard one reads no weights
    assert call(_dims(), gqe.GQE_SLOTS_FULL, os_=None) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_FULL, sw=None) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_WEIGHTED, sw=None) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_WEIGHTED, sw=MIS, os_=None) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(), gqe.GQE_SLOTS_WEIGHTED, T=0, os_=None) == gqe.GQE_OK
    assert call(_dims(), gqe.GQE_SLOTS_HARD, T=0, sw=None, os_=None) == gqe.GQE_OK
    assert call(_dims(D=1 << 23), gqe.GQE_SLOTS_HARD, T=0, sw=None, os_=None) == gqe.GQE_ERR_UNSUPPORTED


def test_out_proj_bwd_validation():
    lib = _lib()

    def call(dims, mode, T=10, sw=A, os_=A, dos=A, ws=A, nbytes=1 << 40):
        n = lambda v: None if v is None else P(v)  # noqa: E731
        return lib.gqe_out_proj_bwd(ctypes.byref(dims), mode, T, P(A), n(sw), n(os_), P(A), P(A), P(A), P(A),
                                    n(dos), P(A), n(ws), nbytes, None)

    assert call(_dims(), 3) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(), gqe.GQE_SLOTS_FULL, T=-1) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_FULL, dos=None) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_FULL, os_=None) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_WEIGHTED, sw=None) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), gqe.GQE_SLOTS_FULL, ws=None) == gqe.GQE_ERR_WORKSPACE
    assert call(_dims(), gqe.GQE_SLOTS_HARD, nbytes=16) == gqe.GQE_ERR_WORKSPACE
    assert call(_dims(), gqe.GQE_SLOTS_WEIGHTED, ws=MIS, os_=None, dos=None) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(), gqe.GQE_SLOTS_HARD, T=0, sw=None, os_=None, dos=None) == gqe.GQE_OK
    # workspace: fp32 dA and the slot vectors A over Kd columns, Kd = (G*k+2)*d for the
    # full layout and G*k*d for the ablation layouts (T=16: one split, no partials)
    r256 = lambda v: (v + 255) // 256 * 256  # noqa: E731
    d = _dims(B=1, S=16, D=64, N=8, G=2, k=2, d=64)
    for mode, kd in ((gqe.GQE_SLOTS_FULL, 6 * 64), (gqe.GQE_SLOTS_HARD, 4 * 64), (gqe.GQE_SLOTS_WEIGHTED, 4 * 64)):
        got = lib.gqe_out_proj_bwd_workspace_bytes(ctypes.byref(d), mode, 16)
        assert got == r256(16 * kd * 4) + r256(16 * kd * 2), (mode, got)


def test_route_bwd_validation():
    lib = _lib()

    def call(dims, weights=gqe.GQE_WEIGHTS_RENORM, aux=0.0, ws=A, dz=None):
        return lib.gqe_route_bwd(ctypes.byref(dims), P(A), P(A), P(A), P(A), P(A), weights, aux,
                                 None if dz is None else P(dz), P(A), P(A), P(A), None, P(ws), 1 << 40, None)

    assert call(_dims(), weights=2) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(), weights=-1) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(), aux=float("nan")) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), aux=-1.0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), aux=float("inf")) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), dz=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(), ws=0) == gqe.GQE_ERR_WORKSPACE
    assert call(_dims(B=0), weights=gqe.GQE_WEIGHTS_PROB, ws=0) == gqe.GQE_OK


def test_qkv_proj_validation():
    lib = _lib()

    def call(dims, x=A, idx=A, q=A, k=A):
        return lib.gqe_qkv_proj(ctypes.byref(dims), P(x), P(A), P(A), P(A), P(idx), P(q), P(k), P(A), None)

    assert call(_dims(N=8, G=3)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(d=96)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(D=96)) == gqe.GQE_ERR_UNSUPPORTED            # bf16 needs D % 64 == 0
    assert call(_dims(), x=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), idx=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), q=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(B=0)) == gqe.GQE_OK
    assert call(_dims(S=0)) == gqe.GQE_OK
    assert call(_dims(B=0, D=96, dtype=gqe.GQE_F32)) == gqe.GQE_OK  # fp32 takes any D % 8


def test_qkv_proj_decode_validation():
    lib = _lib()

    def call(dims, L=1, kv=A, kc=A):
        return lib.gqe_qkv_proj_decode(ctypes.byref(dims), L, P(A), P(A), P(A), P(A), P(A), P(kv), P(A),
                                       P(kc), P(A), None)

    assert call(_dims(), L=-1) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), kv=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), kc=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(S=4), L=5) == gqe.GQE_ERR_INVALID_ARG          # q_len > S_max
    assert call(_dims(D=96)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(N=8, G=3)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(B=0)) == gqe.GQE_OK
    assert call(_dims(), L=0) == gqe.GQE_OK


def test_decode_paged_validation():
    lib = _lib()

    def call(dims, L=1, page=64, bt=A, kvs=None, ws=A, nws=1 << 30):
        return lib.gqe_attn_decode_paged(ctypes.byref(dims), L, P(A), P(A), P(A), P(bt), page,
                                         None if kvs is None else P(kvs), P(A), P(A), P(A), P(A),
                                         None if ws is None else P(ws), nws, None)

    d = _dims(S=4096, N=32, G=8, k=2, d=128)
    assert call(d, page=48) == gqe.GQE_ERR_UNSUPPORTED    # not a power of two
    assert call(d, page=32) == gqe.GQE_ERR_UNSUPPORTED    # below 64
    assert call(_dims(S=4000), page=64) == gqe.GQE_ERR_INVALID_ARG  # S not a multiple of the page
    assert call(d, bt=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(d, kvs=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(d, ws=None) == gqe.GQE_ERR_WORKSPACE
    assert call(d, L=-1) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(S=128, k=2), L=6, page=64) == gqe.GQE_ERR_UNSUPPORTED  # (k+1)*q_len > 16
    assert call(_dims(B=0, S=128), page=64) == gqe.GQE_OK
    assert call(d, L=0) == gqe.GQE_OK


def test_prefill_train_validation():
    lib = _lib()

    def call(dims, q=A, lr=A, ls=A):
        return lib.gqe_attn_prefill_train(ctypes.byref(dims), P(q), P(A), P(A), P(A), P(A), P(A), P(lr), P(ls),
                                          None)

    assert call(_dims(), lr=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), ls=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), lr=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(), q=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(d=96)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(B=0)) == gqe.GQE_OK


def test_prefill_bwd_validation():
    lib = _lib()

    def call(dims, dq=A, do=A, ws=A, nbytes=1 << 40):
        return lib.gqe_attn_prefill_bwd(ctypes.byref(dims), P(A), P(A), P(A), P(A), P(A), P(A), P(A), P(A), P(do),
                                        P(A), P(dq), P(A), P(A), P(ws), nbytes, None)

    assert call(_dims(), dq=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), do=0) == gqe.GQE_ERR_INVALID_ARG
    assert call(_dims(), dq=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(), ws=0) == gqe.GQE_ERR_WORKSPACE
    assert call(_dims(), nbytes=16) == gqe.GQE_ERR_WORKSPACE
    assert call(_dims(), ws=MIS) == gqe.GQE_ERR_ALIGNMENT
    assert call(_dims(N=8, G=3)) == gqe.GQE_ERR_UNSUPPORTED
    assert call(_dims(B=0), ws=0) == gqe.GQE_OK
    assert call(_dims(S=0), ws=0) == gqe.GQE_OK
    # packed rows: B*(G+1)*Rp with Rp = S*k rounded up to 32; bf16 adds 4 fp32 planes of B*S*d
    d = _dims(B=2, S=100, N=8, G=2, k=2, d=64)
    rows = 2 * 3 * 224
    r256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    want = 2 * r256(rows * 64 * 2) + 2 * r256(rows * 4) + r256(4 * 2 * 100 * 64 * 4)
    assert lib.gqe_attn_prefill_bwd_workspace_bytes(ctypes.byref(d)) == want
    d32 = _dims(B=2, S=100, N=8, G=2, k=2, d=64, dtype=gqe.GQE_F32)
    assert lib.gqe_attn_prefill_bwd_workspace_bytes(ctypes.byref(d32)) == 2 * r256(rows * 64 * 4) + 2 * r256(rows * 4)
    assert lib.gqe_attn_prefill_bwd_workspace_bytes(ctypes.byref(_dims(N=8, G=3))) == 0


def test_workspace_sizes_closed_form():
    lib = _lib()
    d = _dims(B=16, S=65536, N=32, G=8, k=2, d=128)
    # split geometry: ~2048 blocks over B*G = 128 pairs -> 16 splits of 4096 keys
    recs = 16 * 8 * 16 * 3
    assert lib.gqe_decode_workspace_bytes(ctypes.byref(d), 1) == recs * (128 + 2) * 4
    # small cache: splits are at least 512 keys -> 2 splits of 1000 keys; q_len=2 -> (k+1)*2 rows
    d3 = _dims(B=1, S=1000, N=4, G=2, k=1, d=64)
    assert lib.gqe_decode_workspace_bytes(ctypes.byref(d3), 2) == (1 * 2 * 2 * 4) * (64 + 2) * 4
    d2 = _dims(B=1, S=131072, N=16, G=8, k=1)
    assert lib.gqe_route_workspace_bytes(ctypes.byref(d2)) == 1 * 8 * 2 * 2048 * 4
    assert lib.gqe_route_workspace_bytes(ctypes.byref(_dims(N=8, G=3))) == 0


def test_binding_rejects_host_tensors():
    import torch
    _lib()
    dims = _dims(B=1, S=4, D=64, N=4, G=2, k=1, d=32, dtype=gqe.GQE_F32)
    x = torch.zeros(4, 64)
    with pytest.raises(ValueError, match="device tensor"):
        gqe.gqe_route(dims, x, torch.zeros(4, 64), None, None, x, x, None, None, None)
    with pytest.raises(ValueError, match="device tensor"):
        gqe.gqe_out_proj_variant(dims, gqe.GQE_SLOTS_HARD, 4, torch.zeros(4, 2, 1, 32), None, None,
                                 torch.zeros(64, 64), torch.zeros(4, 64))
