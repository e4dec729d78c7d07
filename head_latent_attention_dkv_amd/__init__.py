"""Python binding of libmla.so (the MI355X MLA kernels behind a C ABI).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory (tensor data pointers) and the current HIP
stream.  The entry points keep the C names: mla_validate, mla_workspace_bytes,
mla_cache_append, mla_prefill, mla_prefill_chunk, mla_decode, mla_decode_attention,
mla_prefill_attention, mla_status_str, and for compressed convolutional attention
mla_cca_validate, mla_cca_workspace_bytes, mla_cca_prefill.

If the shared library is missing, loading raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmla.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mla.h")

# enums of include/mla.h
MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_SHAPE, MLA_ERR_CAPACITY = 0, 1, 2, 3
MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 4, 5, 6
MLA_DTYPE_F32, MLA_DTYPE_BF16 = 0, 1
MLA_ROPE_NONE, MLA_ROPE_DECOUPLED_INTERLEAVED, MLA_ROPE_FULL_HALFSPLIT = 0, 1, 2
MLA_OP_CACHE_APPEND, MLA_OP_PREFILL, MLA_OP_DECODE = 0, 1, 2
MLA_OP_DECODE_ATTENTION, MLA_OP_PREFILL_ATTENTION, MLA_OP_PREFILL_CHUNK = 3, 4, 5


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {mla_status_str(status)} ({status})")
        self.status = status


class mla_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("d_model", "n_heads", "d_nope", "d_v", "d_rope", "r_kv", "r_q",
                 "n_latent_heads", "rope_mode", "dtype")] + \
               [("rope_base", ctypes.c_float), ("softmax_scale", ctypes.c_float)]


class mla_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_dq", "w_uq", "w_qr", "w_q", "w_dkv", "w_kr", "w_uk", "w_uv", "w_o")]


class mla_cache(ctypes.Structure):
    _fields_ = [("ckv", ctypes.c_void_p), ("kr", ctypes.c_void_p),
                ("max_batch", ctypes.c_int32), ("max_seq", ctypes.c_int32)]


class mla_cca_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("d_model", "n_heads", "n_kv_heads", "head_dim", "num_conv_layers", "conv_kernel_seq",
                 "conv_kernel_ch", "qk_mean", "value_shift", "dtype")] + [("rope_base", ctypes.c_float)]


class mla_cca_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_qk", "w_v", "w_o", "conv_seq", "conv_ch")] + \
               [("key_temperature", ctypes.c_float)]


_lib: Optional[ctypes.CDLL] = None

EXPORTS = ("mla_status_str", "mla_validate", "mla_workspace_bytes", "mla_cache_append",
           "mla_prefill", "mla_decode", "mla_decode_attention", "mla_prefill_attention",
           "mla_prefill_chunk", "mla_cca_validate", "mla_cca_workspace_bytes", "mla_cca_prefill",
           "mla_decode_attention_noalloc", "mla_decode_attention_noalloc_max_bytes", "mla_train_saved_bytes",
           "mla_train_workspace_bytes", "mla_train_forward", "mla_train_backward")

GRAD_ORDER = ("dx", "dw_dq", "dw_uq", "dw_qr", "dw_dkv", "dw_kr", "dw_uk", "dw_uv", "dw_o")


class mla_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_ORDER]


def lib() -> ctypes.CDLL:
    """Load libmla.so (built by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        # PyTorch ships its own HIP runtime under the same soname: load it first so that the
        # library binds to the runtime that owns the tensors and streams handed to it (loaded
        # the other way round, calls fail with MLA_ERR_HIP or launch nothing)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D, W, C = ctypes.POINTER(mla_dims), ctypes.POINTER(mla_weights), ctypes.POINTER(mla_cache)
        L.mla_status_str.restype = ctypes.c_char_p
        L.mla_status_str.argtypes = [ctypes.c_int]
        L.mla_validate.restype = ctypes.c_int
        L.mla_validate.argtypes = [D]
        L.mla_workspace_bytes.restype = sz
        L.mla_workspace_bytes.argtypes = [D, ctypes.c_int, i32, i32]
        L.mla_cache_append.restype = ctypes.c_int
        L.mla_cache_append.argtypes = [D, W, vp, i32, i32, vp, i32, C, vp]
        L.mla_prefill.restype = ctypes.c_int
        L.mla_prefill.argtypes = [D, W, vp, i32, i32, C, vp, vp, sz, vp]
        L.mla_decode.restype = ctypes.c_int
        L.mla_decode.argtypes = [D, W, vp, i32, vp, i32, C, vp, vp, sz, vp]
        L.mla_decode_attention.restype = ctypes.c_int
        L.mla_decode_attention.argtypes = [D, vp, vp, i32, vp, i32, C, vp, vp, sz, vp]
        L.mla_prefill_attention.restype = ctypes.c_int
        L.mla_prefill_attention.argtypes = [D, W, vp, i32, i32, C, vp, vp, sz, vp]
        L.mla_prefill_chunk.restype = ctypes.c_int
        L.mla_prefill_chunk.argtypes = [D, W, vp, i32, i32, i32, C, vp, vp, sz, vp]
        L.mla_decode_attention_noalloc.restype = ctypes.c_int
        L.mla_decode_attention_noalloc.argtypes = [D, vp, vp, i32, vp, i32, C, vp, vp]
        L.mla_decode_attention_noalloc_max_bytes.restype = sz
        L.mla_decode_attention_noalloc_max_bytes.argtypes = []
        L.mla_train_saved_bytes.restype = sz
        L.mla_train_saved_bytes.argtypes = [D, i32, i32]
        L.mla_train_workspace_bytes.restype = sz
        L.mla_train_workspace_bytes.argtypes = [D, i32, i32]
        u64, f32 = ctypes.c_uint64, ctypes.c_float
        L.mla_train_forward.restype = ctypes.c_int
        L.mla_train_forward.argtypes = [D, W, vp, i32, i32, f32, u64, vp, vp, sz, vp]
        L.mla_train_backward.restype = ctypes.c_int
        L.mla_train_backward.argtypes = [D, W, vp, i32, i32, f32, u64, vp, vp, sz, ctypes.POINTER(mla_grads), vp, sz, vp]
        CD, CW = ctypes.POINTER(mla_cca_dims), ctypes.POINTER(mla_cca_weights)
        L.mla_cca_validate.restype = ctypes.c_int
        L.mla_cca_validate.argtypes = [CD]
        L.mla_cca_workspace_bytes.restype = sz
        L.mla_cca_workspace_bytes.argtypes = [CD, i32, i32]
        L.mla_cca_prefill.restype = ctypes.c_int
        L.mla_cca_prefill.argtypes = [CD, CW, vp, i32, i32, vp, vp, sz, vp]
        _lib = L
    return _lib


def mla_status_str(status: int) -> str:
    return lib().mla_status_str(int(status)).decode()


def make_dims(family: str, d_model: int, n_heads: int, d_nope: int, d_rope: int, r_kv: int,
              r_q: int, n_latent_heads: int = 1, dtype: str = "bf16", rope_base: float = 10000.0,
              softmax_scale: float = 0.0) -> mla_dims:
    mode = {"decoupled": MLA_ROPE_DECOUPLED_INTERLEAVED, "fullrope": MLA_ROPE_FULL_HALFSPLIT,
            "mlra": MLA_ROPE_NONE}[family]
    if family == "decoupled" and d_rope == 0:
        mode = MLA_ROPE_NONE
    return mla_dims(d_model, n_heads, d_nope, d_nope, d_rope, r_kv, r_q, n_latent_heads, mode,
                    MLA_DTYPE_BF16 if dtype == "bf16" else MLA_DTYPE_F32, rope_base, softmax_scale)


def dims_from_cfg(cfg) -> mla_dims:
    return make_dims(cfg.family, cfg.d_model, cfg.n_heads, cfg.d_nope, cfg.d_rope, cfg.r_kv,
                     cfg.r_q, cfg.n_latent_heads, cfg.dtype, cfg.rope_base)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def weights_struct(w: Dict[str, object]) -> mla_weights:
    return mla_weights(*[_ptr(w.get(n)) for n in
                         ("w_dq", "w_uq", "w_qr", "w_q", "w_dkv", "w_kr", "w_uk", "w_uv", "w_o")])


def cache_struct(ckv, kr, max_batch: int, max_seq: int) -> mla_cache:
    return mla_cache(_ptr(ckv), _ptr(kr), int(max_batch), int(max_seq))


def _check(status: int, where: str) -> None:
    if status != MLA_OK:
        raise MLAError(status, where)


def mla_validate(dims: mla_dims) -> int:
    return lib().mla_validate(ctypes.byref(dims))


def mla_workspace_bytes(dims: mla_dims, op: int, batch: int, seq_or_max_ctx: int) -> int:
    return lib().mla_workspace_bytes(ctypes.byref(dims), int(op), int(batch), int(seq_or_max_ctx))


def mla_cache_append(dims, weights: mla_weights, x, B: int, T: int, start_pos, max_start: int,
                     cache: mla_cache, stream=None) -> None:
    _check(lib().mla_cache_append(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                                  _ptr(start_pos), int(max_start), ctypes.byref(cache),
                                  _stream(stream)), "mla_cache_append")


def mla_prefill(dims, weights: mla_weights, x, B: int, S: int, cache: Optional[mla_cache], y,
                workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().mla_prefill(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, S,
                             ctypes.byref(cache) if cache is not None else None, _ptr(y),
                             _ptr(workspace), int(ws_bytes), _stream(stream)), "mla_prefill")


def mla_prefill_chunk(dims, weights: mla_weights, x, B: int, T: int, start_pos: int, cache: mla_cache,
                      y, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().mla_prefill_chunk(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                                   int(start_pos), ctypes.byref(cache), _ptr(y), _ptr(workspace),
                                   int(ws_bytes), _stream(stream)), "mla_prefill_chunk")


def mla_decode(dims, weights: mla_weights, x, B: int, ctx_len, max_ctx: int, cache: mla_cache,
               y, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().mla_decode(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, _ptr(ctx_len),
                            int(max_ctx), ctypes.byref(cache), _ptr(y), _ptr(workspace),
                            int(ws_bytes), _stream(stream)), "mla_decode")


def mla_decode_attention(dims, q_lat, q_rope, B: int, ctx_len, max_ctx: int, cache: mla_cache, z,
                         workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().mla_decode_attention(ctypes.byref(dims), _ptr(q_lat), _ptr(q_rope), B,
                                      _ptr(ctx_len), int(max_ctx), ctypes.byref(cache), _ptr(z),
                                      _ptr(workspace), int(ws_bytes), _stream(stream)),
           "mla_decode_attention")


def mla_decode_attention_noalloc(dims, q_lat, q_rope, B: int, ctx_len, max_ctx: int, cache: mla_cache, z,
                                 stream=None) -> None:
    _check(lib().mla_decode_attention_noalloc(ctypes.byref(dims), _ptr(q_lat), _ptr(q_rope), B, _ptr(ctx_len),
                                              int(max_ctx), ctypes.byref(cache), _ptr(z), _stream(stream)),
           "mla_decode_attention_noalloc")


def mla_decode_attention_noalloc_max_bytes() -> int:
    return int(lib().mla_decode_attention_noalloc_max_bytes())


def mla_prefill_attention(dims, weights: mla_weights, q, B: int, S: int, cache: mla_cache, o,
                          workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().mla_prefill_attention(ctypes.byref(dims), ctypes.byref(weights), _ptr(q), B, S,
                                       ctypes.byref(cache), _ptr(o), _ptr(workspace),
                                       int(ws_bytes), _stream(stream)), "mla_prefill_attention")


def mla_train_saved_bytes(dims, B: int, S: int) -> int:
    return int(lib().mla_train_saved_bytes(ctypes.byref(dims), int(B), int(S)))


def mla_train_workspace_bytes(dims, B: int, S: int) -> int:
    return int(lib().mla_train_workspace_bytes(ctypes.byref(dims), int(B), int(S)))


def mla_train_forward(dims, weights: mla_weights, x, B: int, S: int, dropout_p: float, seed: int, y, saved,
                      saved_bytes: int, stream=None) -> None:
    _check(lib().mla_train_forward(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, S, float(dropout_p),
                                   int(seed), _ptr(y), _ptr(saved), int(saved_bytes), _stream(stream)),
           "mla_train_forward")


def grads_struct(g: Dict[str, object]) -> mla_grads:
    return mla_grads(*[_ptr(g.get(n)) for n in GRAD_ORDER])


def mla_train_backward(dims, weights: mla_weights, x, B: int, S: int, dropout_p: float, seed: int, dy, saved,
                       saved_bytes: int, grads: mla_grads, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().mla_train_backward(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, S, float(dropout_p),
                                    int(seed), _ptr(dy), _ptr(saved), int(saved_bytes), ctypes.byref(grads),
                                    _ptr(workspace), int(ws_bytes), _stream(stream)), "mla_train_backward")


def cca_dims_from_cfg(cfg) -> mla_cca_dims:
    return mla_cca_dims(cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.num_conv_layers,
                        cfg.conv_kernel_seq, cfg.conv_kernel_ch, int(cfg.qk_mean), int(cfg.value_shift),
                        MLA_DTYPE_BF16 if cfg.dtype == "bf16" else MLA_DTYPE_F32, cfg.rope_base)


def cca_weights_struct(w: Dict[str, object], key_temperature: float) -> mla_cca_weights:
    return mla_cca_weights(*[_ptr(w.get(n)) for n in ("w_qk", "w_v", "w_o", "conv_seq", "conv_ch")],
                           float(key_temperature))


def mla_cca_validate(dims: mla_cca_dims) -> int:
    return lib().mla_cca_validate(ctypes.byref(dims))


def mla_cca_workspace_bytes(dims: mla_cca_dims, B: int, S: int) -> int:
    return lib().mla_cca_workspace_bytes(ctypes.byref(dims), int(B), int(S))


def mla_cca_prefill(dims, weights: mla_cca_weights, x, B: int, S: int, y, workspace, ws_bytes: int,
                    stream=None) -> None:
    _check(lib().mla_cca_prefill(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, S, _ptr(y),
                                 _ptr(workspace), int(ws_bytes), _stream(stream)), "mla_cca_prefill")


__all__ = [n for n in dir() if n.startswith(("mla_", "MLA_"))] + [
    "cca_dims_from_cfg", "cca_weights_struct", "grads_struct", "GRAD_ORDER", 
    "lib", "make_dims", "dims_from_cfg", "weights_struct", "cache_struct", "MLAError",
    "LIB_PATH", "HEADER_PATH", "EXPORTS"]
