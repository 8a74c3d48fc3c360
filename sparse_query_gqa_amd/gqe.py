"""Thin ctypes binding of libgqe.so (include/gqe.h).

The ``gqe_*`` functions have the C ABI's names and arguments; they only
check that the tensors match the declared shapes/dtypes, pass device
pointers and the current HIP stream, and turn a non-zero status into
``GQEError``. Every step of the layer runs in the library's HIP kernels;
there is no other code path. ``route``/``prefill``/``decode``/``out_proj``
additionally allocate their outputs with torch.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# GQE_LIB names another build of the same library (the host-sanitizer build
# the CPU tests load); by default the in-tree libgqe.so
LIB_PATH = os.environ.get("GQE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqe.so")

GQE_OK = 0
GQE_ERR_INVALID_ARG = -1
GQE_ERR_UNSUPPORTED = -2
GQE_ERR_ALIGNMENT = -3
GQE_ERR_WORKSPACE = -4
GQE_ERR_HIP = -5
GQE_ERR_SCRATCH = -6
GQE_BF16 = 0
GQE_F32 = 1
GQE_SLOTS_FULL = 0
GQE_SLOTS_HARD = 1
GQE_SLOTS_WEIGHTED = 2
GQE_WEIGHTS_RENORM = 0
GQE_WEIGHTS_PROB = 1

EXPORTED = [
    "gqe_status_string", "gqe_version", "gqe_route_workspace_bytes", "gqe_route",
    "gqe_attn_prefill", "gqe_decode_workspace_bytes", "gqe_attn_decode", "gqe_out_proj",
    "gqe_qkv_proj", "gqe_qkv_proj_decode", "gqe_attn_decode_paged", "gqe_out_proj_variant",
    "gqe_attn_prefill_train", "gqe_attn_prefill_bwd_workspace_bytes", "gqe_attn_prefill_bwd",
    "gqe_out_proj_bwd_workspace_bytes", "gqe_out_proj_bwd", "gqe_route_bwd_workspace_bytes", "gqe_route_bwd",
    "gqe_decode_scratch_bytes", "gqe_attn_decode_noalloc",
]


class GQEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class gqe_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "S", "D", "N", "G", "k", "d", "dtype")]

    @classmethod
    def make(cls, B, S, D, N, G, k, d, dtype) -> "gqe_dims":
        code = {"bf16": GQE_BF16, torch.bfloat16: GQE_BF16, "f32": GQE_F32,
                torch.float32: GQE_F32}.get(dtype, dtype)
        return cls(B, S, D, N, G, k, d, code)

    @classmethod
    def from_config(cls, cfg) -> "gqe_dims":
        return cls.make(cfg.B, cfg.S, cfg.D, cfg.N, cfg.G, cfg.k, cfg.d, cfg.dtype)

    @property
    def M(self) -> int:
        return self.N // self.G

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == GQE_BF16 else torch.float32


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgqe.so; raises when it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_query_gqa_amd.build`"
                           " (the GQE layer has no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(gqe_dims)
    sig = {
        "gqe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "gqe_version": (ctypes.c_int, []),
        "gqe_route_workspace_bytes": (SZ, [D]),
        "gqe_route": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "gqe_attn_prefill": (ctypes.c_int, [D, P, P, P, P, P, P, P]),
        "gqe_decode_workspace_bytes": (SZ, [D, I32]),
        "gqe_attn_decode": (ctypes.c_int, [D, I32, P, P, P, P, P, P, P, P, SZ, P]),
        "gqe_decode_scratch_bytes": (SZ, []),
        "gqe_attn_decode_noalloc": (ctypes.c_int, [D, I32, P, P, P, P, P, P, P, P]),
        "gqe_out_proj": (ctypes.c_int, [D, I64, P, P, P, P, P, P]),
        "gqe_qkv_proj": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P]),
        "gqe_qkv_proj_decode": (ctypes.c_int, [D, I32, P, P, P, P, P, P, P, P, P, P]),
        "gqe_attn_decode_paged": (ctypes.c_int, [D, I32, P, P, P, P, I32, P, P, P, P, P, P, SZ, P]),
        "gqe_out_proj_variant": (ctypes.c_int, [D, I32, I64, P, P, P, P, P, P]),
        "gqe_attn_prefill_train": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P]),
        "gqe_attn_prefill_bwd_workspace_bytes": (SZ, [D]),
        "gqe_attn_prefill_bwd": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "gqe_out_proj_bwd_workspace_bytes": (SZ, [D, I32, I64]),
        "gqe_out_proj_bwd": (ctypes.c_int, [D, I32, I64, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "gqe_route_bwd_workspace_bytes": (SZ, [D]),
        "gqe_route_bwd": (ctypes.c_int, [D, P, P, P, P, P, I32, ctypes.c_float, P, P, P, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().gqe_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _check(t: Optional[torch.Tensor], name: str, shape, dtype, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(st: int, where: str):
    if st != GQE_OK:
        raise GQEError(st, where)


def gqe_route_workspace_bytes(dims: gqe_dims) -> int:
    return load_library().gqe_route_workspace_bytes(ctypes.byref(dims))


def gqe_decode_workspace_bytes(dims: gqe_dims, q_len: int) -> int:
    return load_library().gqe_decode_workspace_bytes(ctypes.byref(dims), q_len)


def gqe_route(dims, x, w_router, b_router, logits, topk_idx, topk_w, list_off, list_tok,
              workspace, stream=None, topk_p=None):
    T, GM, G, k, dt = dims.B * dims.S, dims.N, dims.G, dims.k, dims.torch_dtype
    _check(x, "x", (T, dims.D), dt)
    _check(w_router, "w_router", (GM, dims.D), dt)
    _check(b_router, "b_router", (GM,), torch.float32, optional=True)
    _check(logits, "logits", (T, G, dims.M), torch.float32, optional=True)
    _check(topk_idx, "topk_idx", (T, G, k), torch.int32)
    _check(topk_w, "topk_w", (T, G, k), torch.float32)
    _check(topk_p, "topk_p", (T, G, k), torch.float32, optional=True)
    _check(list_off, "list_off", (dims.B, G, dims.M + 1), torch.int32, optional=True)
    _check(list_tok, "list_tok", (dims.B, G, k * dims.S), torch.int32, optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().gqe_route(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(b_router),
                                  _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(topk_p),
                                  _ptr(list_off), _ptr(list_tok), _ptr(workspace), ws_bytes,
                                  _stream(stream))
    _raise(st, "gqe_route")


def gqe_attn_prefill(dims, q, k, v, topk_idx, o_routed, o_shared, stream=None):
    B, S, N, G, kk, d, dt = dims.B, dims.S, dims.N, dims.G, dims.k, dims.d, dims.torch_dtype
    _check(q, "q", (B, S, N + 1, d), dt)
    _check(k, "k", (B, G, S, d), dt)
    _check(v, "v", (B, G, S, d), dt)
    _check(topk_idx, "topk_idx", (B * S, G, kk), torch.int32)
    _check(o_routed, "o_routed", (B, S, G, kk, d), dt)
    _check(o_shared, "o_shared", (B, S, d), dt)
    st = load_library().gqe_attn_prefill(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(topk_idx), _ptr(o_routed), _ptr(o_shared),
                                         _stream(stream))
    _raise(st, "gqe_attn_prefill")


def gqe_attn_prefill_train(dims, q, k, v, topk_idx, o_routed, o_shared, lse_routed, lse_shared,
                           stream=None):
    B, S, N, G, kk, d, dt = dims.B, dims.S, dims.N, dims.G, dims.k, dims.d, dims.torch_dtype
    _check(q, "q", (B, S, N + 1, d), dt)
    _check(k, "k", (B, G, S, d), dt)
    _check(v, "v", (B, G, S, d), dt)
    _check(topk_idx, "topk_idx", (B * S, G, kk), torch.int32)
    _check(o_routed, "o_routed", (B, S, G, kk, d), dt)
    _check(o_shared, "o_shared", (B, S, d), dt)
    _check(lse_routed, "lse_routed", (B, S, G, kk), torch.float32)
    _check(lse_shared, "lse_shared", (B, S), torch.float32)
    st = load_library().gqe_attn_prefill_train(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(topk_idx), _ptr(o_routed), _ptr(o_shared),
                                               _ptr(lse_routed), _ptr(lse_shared), _stream(stream))
    _raise(st, "gqe_attn_prefill_train")


def gqe_attn_prefill_bwd_workspace_bytes(dims: gqe_dims) -> int:
    return load_library().gqe_attn_prefill_bwd_workspace_bytes(ctypes.byref(dims))


def gqe_attn_prefill_bwd(dims, q, k, v, topk_idx, o_routed, o_shared, lse_routed, lse_shared,
                         do_routed, do_shared, dq, dk, dv, workspace, stream=None):
    B, S, N, G, kk, d, dt = dims.B, dims.S, dims.N, dims.G, dims.k, dims.d, dims.torch_dtype
    for t, name, shape in ((q, "q", (B, S, N + 1, d)), (k, "k", (B, G, S, d)), (v, "v", (B, G, S, d)),
                           (o_routed, "o_routed", (B, S, G, kk, d)), (o_shared, "o_shared", (B, S, d)),
                           (do_routed, "do_routed", (B, S, G, kk, d)), (do_shared, "do_shared", (B, S, d)),
                           (dq, "dq", (B, S, N + 1, d)), (dk, "dk", (B, G, S, d)), (dv, "dv", (B, G, S, d))):
        _check(t, name, shape, dt)
    _check(topk_idx, "topk_idx", (B * S, G, kk), torch.int32)
    _check(lse_routed, "lse_routed", (B, S, G, kk), torch.float32)
    _check(lse_shared, "lse_shared", (B, S), torch.float32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().gqe_attn_prefill_bwd(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(o_routed), _ptr(o_shared),
        _ptr(lse_routed), _ptr(lse_shared), _ptr(do_routed), _ptr(do_shared), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), ws_bytes, _stream(stream))
    _raise(st, "gqe_attn_prefill_bwd")


def _slot_rows(dims, mode) -> int:
    """W_O rows: [O, obar, s] for the full layout, the hard slots alone for the ablation layouts."""
    return (dims.G * dims.k + (2 if mode == GQE_SLOTS_FULL else 0)) * dims.d


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def gqe_out_proj_bwd_workspace_bytes(dims, mode, T) -> int:
    return load_library().gqe_out_proj_bwd_workspace_bytes(ctypes.byref(dims), int(mode), int(T))


def gqe_out_proj_bwd(dims, mode, T, o_routed, slot_w, o_shared, w_o, dy, do_routed, dw, do_shared, dw_o,
                     workspace, stream=None):
    G, kk, d, D, dt = dims.G, dims.k, dims.d, dims.D, dims.torch_dtype
    full = mode == GQE_SLOTS_FULL
    _check(o_routed, "o_routed", (T, G, kk, d), dt)
    _check(slot_w, "slot_w", (T, G, kk), torch.float32, optional=mode == GQE_SLOTS_HARD)
    _check(o_shared, "o_shared", (T, d), dt, optional=not full)
    _check(w_o, "w_o", (_slot_rows(dims, mode), D), dt)
    _check(dy, "dy", (T, D), dt)
    _check(do_routed, "do_routed", (T, G, kk, d), dt)
    _check(dw, "dw", (T, G, kk), torch.float32)
    _check(do_shared, "do_shared", (T, d), dt, optional=not full)
    _check(dw_o, "dw_o", (_slot_rows(dims, mode), D), torch.float32)
    st = load_library().gqe_out_proj_bwd(ctypes.byref(dims), int(mode), int(T), _ptr(o_routed), _ptr(slot_w),
                                         _ptr(o_shared), _ptr(w_o), _ptr(dy), _ptr(do_routed), _ptr(dw),
                                         _ptr(do_shared), _ptr(dw_o), _ptr(workspace), _nbytes(workspace),
                                         _stream(stream))
    _raise(st, "gqe_out_proj_bwd")


def gqe_route_bwd_workspace_bytes(dims) -> int:
    return load_library().gqe_route_bwd_workspace_bytes(ctypes.byref(dims))


def gqe_route_bwd(dims, x, w_router, logits, topk_idx, dw, aux_coef, dz, dx, dw_router, db_router, aux_loss,
                  workspace, stream=None, weights=GQE_WEIGHTS_RENORM):
    T, D, G, M, kk, dt = dims.B * dims.S, dims.D, dims.G, dims.M, dims.k, dims.torch_dtype
    _check(x, "x", (T, D), dt)
    _check(w_router, "w_router", (G * M, D), dt)
    _check(logits, "logits", (T, G, M), torch.float32)
    _check(topk_idx, "topk_idx", (T, G, kk), torch.int32)
    _check(dw, "dw", (T, G, kk), torch.float32)
    _check(dz, "dz", (T, G, M), torch.float32, optional=True)
    _check(dx, "dx", (T, D), dt)
    _check(dw_router, "dw_router", (G * M, D), torch.float32)
    _check(db_router, "db_router", (G * M,), torch.float32)
    _check(aux_loss, "aux_loss", (1,), torch.float32, optional=True)
    st = load_library().gqe_route_bwd(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(logits), _ptr(topk_idx),
                                      _ptr(dw), int(weights), float(aux_coef), _ptr(dz), _ptr(dx), _ptr(dw_router),
                                      _ptr(db_router), _ptr(aux_loss), _ptr(workspace), _nbytes(workspace),
                                      _stream(stream))
    _raise(st, "gqe_route_bwd")


def gqe_attn_decode(dims, q_len, q, k_cache, v_cache, kv_len, topk_idx, o_routed, o_shared,
                    workspace, stream=None):
    B, S, N, G, kk, d, dt = dims.B, dims.S, dims.N, dims.G, dims.k, dims.d, dims.torch_dtype
    _check(q, "q", (B, q_len, N + 1, d), dt)
    _check(k_cache, "k_cache", (B, G, S, d), dt)
    _check(v_cache, "v_cache", (B, G, S, d), dt)
    _check(kv_len, "kv_len", (B,), torch.int32)
    _check(topk_idx, "topk_idx", (B * q_len, G, kk), torch.int32)
    _check(o_routed, "o_routed", (B, q_len, G, kk, d), dt)
    _check(o_shared, "o_shared", (B, q_len, d), dt)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().gqe_attn_decode(ctypes.byref(dims), q_len, _ptr(q), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(kv_len), _ptr(topk_idx),
                                        _ptr(o_routed), _ptr(o_shared), _ptr(workspace), ws_bytes,
                                        _stream(stream))
    _raise(st, "gqe_attn_decode")


def gqe_decode_scratch_bytes() -> int:
    return load_library().gqe_decode_scratch_bytes()


def gqe_attn_decode_noalloc(dims, q_len, q, k_cache, v_cache, kv_len, topk_idx, o_routed, o_shared,
                            stream=None):
    """gqe_attn_decode with the split partials in the library's static device scratch (no workspace)."""
    B, S, N, G, kk, d, dt = dims.B, dims.S, dims.N, dims.G, dims.k, dims.d, dims.torch_dtype
    _check(q, "q", (B, q_len, N + 1, d), dt)
    _check(k_cache, "k_cache", (B, G, S, d), dt)
    _check(v_cache, "v_cache", (B, G, S, d), dt)
    _check(kv_len, "kv_len", (B,), torch.int32)
    _check(topk_idx, "topk_idx", (B * q_len, G, kk), torch.int32)
    _check(o_routed, "o_routed", (B, q_len, G, kk, d), dt)
    _check(o_shared, "o_shared", (B, q_len, d), dt)
    st = load_library().gqe_attn_decode_noalloc(ctypes.byref(dims), q_len, _ptr(q), _ptr(k_cache),
                                                _ptr(v_cache), _ptr(kv_len), _ptr(topk_idx),
                                                _ptr(o_routed), _ptr(o_shared), _stream(stream))
    _raise(st, "gqe_attn_decode_noalloc")


def gqe_attn_decode_paged(dims, q_len, q, k_pages, v_pages, block_table, page_size, kv_start, kv_len,
                          topk_idx, o_routed, o_shared, workspace, stream=None):
    B, S, N, G, kk, d, dt = dims.B, dims.S, dims.N, dims.G, dims.k, dims.d, dims.torch_dtype
    _check(q, "q", (B, q_len, N + 1, d), dt)
    if k_pages.dim() != 4 or tuple(k_pages.shape[1:]) != (G, page_size, d):
        raise ValueError(f"k_pages has shape {tuple(k_pages.shape)}, expected (n_pages, {G}, {page_size}, {d})")
    _check(k_pages, "k_pages", tuple(k_pages.shape), dt)
    _check(v_pages, "v_pages", tuple(k_pages.shape), dt)
    _check(block_table, "block_table", (B, S // page_size), torch.int32)
    _check(kv_start, "kv_start", (B,), torch.int32, optional=True)
    _check(kv_len, "kv_len", (B,), torch.int32)
    _check(topk_idx, "topk_idx", (B * q_len, G, kk), torch.int32)
    _check(o_routed, "o_routed", (B, q_len, G, kk, d), dt)
    _check(o_shared, "o_shared", (B, q_len, d), dt)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().gqe_attn_decode_paged(ctypes.byref(dims), q_len, _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                              _ptr(block_table), page_size, _ptr(kv_start), _ptr(kv_len),
                                              _ptr(topk_idx), _ptr(o_routed), _ptr(o_shared), _ptr(workspace),
                                              ws_bytes, _stream(stream))
    _raise(st, "gqe_attn_decode_paged")


def gqe_out_proj_variant(dims, mode, T, o_routed, slot_w, o_shared, w_o, y, stream=None):
    """slot_w: topk_w for the full layout, topk_p for the weighted one, None allowed for the hard one;
    o_shared: read by the full layout only (None allowed otherwise)."""
    G, kk, d, D, dt = dims.G, dims.k, dims.d, dims.D, dims.torch_dtype
    _check(o_routed, "o_routed", (T, G, kk, d), dt)
    _check(slot_w, "slot_w", (T, G, kk), torch.float32, optional=mode == GQE_SLOTS_HARD)
    _check(o_shared, "o_shared", (T, d), dt, optional=mode != GQE_SLOTS_FULL)
    _check(w_o, "w_o", (_slot_rows(dims, mode), D), dt)
    _check(y, "y", (T, D), dt)
    st = load_library().gqe_out_proj_variant(ctypes.byref(dims), mode, T, _ptr(o_routed), _ptr(slot_w),
                                             _ptr(o_shared), _ptr(w_o), _ptr(y), _stream(stream))
    _raise(st, "gqe_out_proj_variant")


def gqe_out_proj(dims, T, o_routed, topk_w, o_shared, w_o, y, stream=None):
    G, kk, d, D, dt = dims.G, dims.k, dims.d, dims.D, dims.torch_dtype
    _check(o_routed, "o_routed", (T, G, kk, d), dt)
    _check(topk_w, "topk_w", (T, G, kk), torch.float32)
    _check(o_shared, "o_shared", (T, d), dt)
    _check(w_o, "w_o", ((G * kk + 2) * d, D), dt)
    _check(y, "y", (T, D), dt)
    st = load_library().gqe_out_proj(ctypes.byref(dims), T, _ptr(o_routed), _ptr(topk_w),
                                     _ptr(o_shared), _ptr(w_o), _ptr(y), _stream(stream))
    _raise(st, "gqe_out_proj")


def gqe_qkv_proj(dims, x, w_q, w_k, w_v, topk_idx, q, k, v, stream=None):
    B, S, D, N, G, kk, d, dt = dims.B, dims.S, dims.D, dims.N, dims.G, dims.k, dims.d, dims.torch_dtype
    _check(x, "x", (B, S, D), dt)
    _check(w_q, "w_q", ((N + 1) * d, D), dt)
    _check(w_k, "w_k", (G * d, D), dt)
    _check(w_v, "w_v", (G * d, D), dt)
    _check(topk_idx, "topk_idx", (B * S, G, kk), torch.int32)
    _check(q, "q", (B, S, N + 1, d), dt)
    _check(k, "k", (B, G, S, d), dt)
    _check(v, "v", (B, G, S, d), dt)
    st = load_library().gqe_qkv_proj(ctypes.byref(dims), _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                     _ptr(topk_idx), _ptr(q), _ptr(k), _ptr(v), _stream(stream))
    _raise(st, "gqe_qkv_proj")


def gqe_qkv_proj_decode(dims, q_len, x, w_q, w_k, w_v, topk_idx, kv_len, q, k_cache, v_cache,
                        stream=None):
    B, S, D, N, G, kk, d, dt = dims.B, dims.S, dims.D, dims.N, dims.G, dims.k, dims.d, dims.torch_dtype
    _check(x, "x", (B, q_len, D), dt)
    _check(w_q, "w_q", ((N + 1) * d, D), dt)
    _check(w_k, "w_k", (G * d, D), dt)
    _check(w_v, "w_v", (G * d, D), dt)
    _check(topk_idx, "topk_idx", (B * q_len, G, kk), torch.int32)
    _check(kv_len, "kv_len", (B,), torch.int32)
    _check(q, "q", (B, q_len, N + 1, d), dt)
    _check(k_cache, "k_cache", (B, G, S, d), dt)
    _check(v_cache, "v_cache", (B, G, S, d), dt)
    st = load_library().gqe_qkv_proj_decode(ctypes.byref(dims), q_len, _ptr(x), _ptr(w_q), _ptr(w_k),
                                            _ptr(w_v), _ptr(topk_idx), _ptr(kv_len), _ptr(q),
                                            _ptr(k_cache), _ptr(v_cache), _stream(stream))
    _raise(st, "gqe_qkv_proj_decode")


# --------------------------------------------------------------------------
# Allocating wrappers
# --------------------------------------------------------------------------

def route(dims, x, w_router, b_router=None, want_logits=True, want_lists=True, stream=None, want_p=False):
    dev = x.device
    T, G, M, k = dims.B * dims.S, dims.G, dims.M, dims.k
    out = dict(
        logits=torch.empty((T, G, M), dtype=torch.float32, device=dev) if want_logits else None,
        topk_idx=torch.empty((T, G, k), dtype=torch.int32, device=dev),
        topk_w=torch.empty((T, G, k), dtype=torch.float32, device=dev),
        topk_p=torch.empty((T, G, k), dtype=torch.float32, device=dev) if want_p else None,
        list_off=torch.empty((dims.B, G, M + 1), dtype=torch.int32, device=dev) if want_lists else None,
        list_tok=torch.empty((dims.B, G, k * dims.S), dtype=torch.int32, device=dev) if want_lists else None,
    )
    ws = None
    if want_lists:
        nbytes = gqe_route_workspace_bytes(dims)
        ws = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=dev)
    gqe_route(dims, x, w_router, b_router, out["logits"], out["topk_idx"], out["topk_w"],
              out["list_off"], out["list_tok"], ws, stream, topk_p=out["topk_p"])
    return out


def prefill(dims, q, k, v, topk_idx, stream=None):
    o_r = torch.empty((dims.B, dims.S, dims.G, dims.k, dims.d), dtype=q.dtype, device=q.device)
    o_s = torch.empty((dims.B, dims.S, dims.d), dtype=q.dtype, device=q.device)
    gqe_attn_prefill(dims, q, k, v, topk_idx, o_r, o_s, stream)
    return o_r, o_s


def prefill_train(dims, q, k, v, topk_idx, stream=None):
    """Forward that also returns each row's log-sum-exp: (o_r, o_s, lse_r, lse_s)."""
    o_r, o_s = (torch.empty(s, dtype=q.dtype, device=q.device)
                for s in ((dims.B, dims.S, dims.G, dims.k, dims.d), (dims.B, dims.S, dims.d)))
    lse_r = torch.empty((dims.B, dims.S, dims.G, dims.k), dtype=torch.float32, device=q.device)
    lse_s = torch.empty((dims.B, dims.S), dtype=torch.float32, device=q.device)
    gqe_attn_prefill_train(dims, q, k, v, topk_idx, o_r, o_s, lse_r, lse_s, stream)
    return o_r, o_s, lse_r, lse_s


def prefill_bwd(dims, q, k, v, topk_idx, o_r, o_s, lse_r, lse_s, do_r, do_s, workspace=None, stream=None):
    """Attention backward: (dq, dk, dv); dq is zero in the rows of unselected heads."""
    if workspace is None:
        workspace = torch.empty((max(gqe_attn_prefill_bwd_workspace_bytes(dims), 16),), dtype=torch.uint8,
                                device=q.device)
    dq = torch.zeros_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    gqe_attn_prefill_bwd(dims, q, k, v, topk_idx, o_r, o_s, lse_r, lse_s, do_r, do_s, dq, dk, dv, workspace,
                         stream)
    return dq, dk, dv


def _workspace(nbytes, device):
    return torch.empty((max(int(nbytes), 16),), dtype=torch.uint8, device=device)


def out_proj_bwd(dims, T, o_routed, slot_w, o_shared, w_o, dy, mode=GQE_SLOTS_FULL, stream=None):
    """Output-projection backward: (do_r [T,G,k,d], dw [T,G,k], do_s [T,d], dw_o fp32).
    slot_w and o_shared as for gqe_out_proj_variant; do_s is zero in the ablation layouts."""
    dev = dy.device
    o_routed = o_routed.reshape(T, dims.G, dims.k, dims.d)
    slot_w = None if slot_w is None else slot_w.reshape(T, dims.G, dims.k)
    o_shared = None if o_shared is None else o_shared.reshape(T, dims.d)
    do_r = torch.empty_like(o_routed)
    dw = torch.empty((T, dims.G, dims.k), dtype=torch.float32, device=dev)
    do_s = torch.empty((T, dims.d), dtype=o_routed.dtype, device=dev)
    dw_o = torch.empty(tuple(w_o.shape), dtype=torch.float32, device=dev)
    ws = _workspace(gqe_out_proj_bwd_workspace_bytes(dims, mode, T), dev)
    gqe_out_proj_bwd(dims, mode, T, o_routed, slot_w, o_shared, w_o, dy, do_r, dw, do_s, dw_o, ws, stream)
    return do_r, dw, do_s, dw_o


def route_bwd(dims, x, w_router, logits, topk_idx, dw, aux_coef=0.0, stream=None, weights=GQE_WEIGHTS_RENORM):
    """Router backward: dict(dz, dx, dw_router, db_router, aux_loss). weights says whether dw is the
    gradient of the renormalised weights (GQE_WEIGHTS_RENORM) or of the selected p (GQE_WEIGHTS_PROB)."""
    dev = x.device
    T, GM = dims.B * dims.S, dims.N
    out = dict(dz=torch.empty((T, dims.G, dims.M), dtype=torch.float32, device=dev), dx=torch.empty_like(x),
               dw_router=torch.empty((GM, dims.D), dtype=torch.float32, device=dev),
               db_router=torch.empty((GM,), dtype=torch.float32, device=dev),
               aux_loss=torch.zeros((1,), dtype=torch.float32, device=dev))
    ws = _workspace(gqe_route_bwd_workspace_bytes(dims), dev)
    gqe_route_bwd(dims, x, w_router, logits, topk_idx, dw, aux_coef, out["dz"], out["dx"], out["dw_router"],
                  out["db_router"], out["aux_loss"], ws, stream, weights=weights)
    return out


def decode_workspace(dims, q_len, device) -> torch.Tensor:
    nbytes = gqe_decode_workspace_bytes(dims, q_len)
    return torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=device)


def decode(dims, q_len, q, k_cache, v_cache, kv_len, topk_idx, workspace=None, stream=None):
    if workspace is None:
        workspace = decode_workspace(dims, q_len, q.device)
    o_r = torch.empty((dims.B, q_len, dims.G, dims.k, dims.d), dtype=q.dtype, device=q.device)
    o_s = torch.empty((dims.B, q_len, dims.d), dtype=q.dtype, device=q.device)
    gqe_attn_decode(dims, q_len, q, k_cache, v_cache, kv_len, topk_idx, o_r, o_s, workspace, stream)
    return o_r, o_s


def qkv_proj(dims, x, w_q, w_k, w_v, topk_idx, q=None, stream=None):
    """Prefill projections; q (if given) keeps the rows of unselected heads."""
    dev, dt = x.device, x.dtype
    if q is None:
        q = torch.zeros((dims.B, dims.S, dims.N + 1, dims.d), dtype=dt, device=dev)
    k = torch.empty((dims.B, dims.G, dims.S, dims.d), dtype=dt, device=dev)
    v = torch.empty((dims.B, dims.G, dims.S, dims.d), dtype=dt, device=dev)
    gqe_qkv_proj(dims, x, w_q, w_k, w_v, topk_idx, q, k, v, stream)
    return q, k, v


def decode_paged(dims, q_len, q, k_pages, v_pages, block_table, page_size, kv_len, topk_idx, kv_start=None,
                 workspace=None, stream=None):
    if workspace is None:
        workspace = decode_workspace(dims, q_len, q.device)
    o_r = torch.empty((dims.B, q_len, dims.G, dims.k, dims.d), dtype=q.dtype, device=q.device)
    o_s = torch.empty((dims.B, q_len, dims.d), dtype=q.dtype, device=q.device)
    gqe_attn_decode_paged(dims, q_len, q, k_pages, v_pages, block_table, page_size, kv_start, kv_len,
                          topk_idx, o_r, o_s, workspace, stream)
    return o_r, o_s


def out_proj(dims, T, o_routed, topk_w, o_shared, w_o, stream=None):
    y = torch.empty((T, dims.D), dtype=w_o.dtype, device=w_o.device)
    gqe_out_proj(dims, T, o_routed.view(T, dims.G, dims.k, dims.d), topk_w.view(T, dims.G, dims.k),
                 o_shared.view(T, dims.d), w_o, y, stream)
    return y
