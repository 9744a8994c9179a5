"""Python binding of libtq (TurboQuant compression, decode attention, search on MI355X).

Argument marshalling only: every function forwards to the C entry point of
the same name in the in-tree ``libtq.so`` (declared in ``include/tq.h``).
Tensors are passed as device pointers (``tensor.data_ptr()``); the stream is
torch's current stream unless one is given. Nothing here computes any step
of the method, and there is no fallback: if the library is not built the
import of a function fails with an error naming the build command.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int64, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY names another build of the same library (the tests run the C ABI
# checks against a host-sanitized build this way); the default is the in-tree one
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(_HERE, "libtq.so")

TQ_OK = 0
TQ_ERR_INVALID_ARG = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_MISALIGNED = -3
TQ_ERR_NO_CONVERGE = -4
TQ_ERR_HIP = -5
TQ_ERR_WORKSPACE = -6
TQ_ERR_SCRATCH = -7
TQ_DECODE_SCRATCH_BYTES = 16 << 20

TQ_MSE, TQ_PROD = 0, 1
TQ_F32, TQ_BF16 = 0, 1
TQ_LAYOUT_KEYS, TQ_LAYOUT_VALUES = 0, 1
TQ_KV_UNIFORM, TQ_KV_ASYMMETRIC, TQ_KV_MIXED = 0, 1, 2
TQ_MAX_LEVELS = 16
TQ_MAX_GROUPS = 4

EXPORTS = [
    "tq_build_codebook", "tq_quantizer_init", "tq_packed_bytes", "tq_status_string",
    "tq_quantize_kv", "tq_append_kv", "tq_append_kv_pair", "tq_decode_workspace_bytes", "tq_decode_attn", "tq_kv_bit_allocation",
    "tq_decode_paged_workspace_bytes", "tq_decode_attn_paged", "tq_decode_attn_noalloc", "tq_decode_step",
    "tq_search_workspace_bytes", "tq_search_topk", "tq_fold_bytes", "tq_fold_qjl",
]


class tq_quantizer(ctypes.Structure):
    _fields_ = [
        ("d", c_int), ("mse_bits", c_int), ("variant", c_int),
        ("R", c_void_p), ("S", c_void_p), ("SR", c_void_p),
        ("centroids", c_float * TQ_MAX_LEVELS), ("thresholds", c_float * (TQ_MAX_LEVELS - 1)),
    ]


class tq_group(ctypes.Structure):
    _fields_ = [
        ("q", tq_quantizer), ("ch_offset", c_int),
        ("packed", c_void_p), ("norm", c_void_p), ("rnorm", c_void_p),
        ("seq_stride", c_int64),
    ]


class tq_kv_desc(ctypes.Structure):
    _fields_ = [("n_groups", c_int), ("g", tq_group * TQ_MAX_GROUPS)]


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {tq_status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree libtq.so (built by ``python -m decode_tq_quantize_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run: python -m decode_tq_quantize_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.tq_build_codebook.argtypes = [c_int, c_int, POINTER(c_double), POINTER(c_double), POINTER(c_double), c_int]
        L.tq_build_codebook.restype = c_int
        L.tq_quantizer_init.argtypes = [POINTER(tq_quantizer), c_int, c_int, c_int, c_void_p, c_void_p]
        L.tq_quantizer_init.restype = c_int
        L.tq_packed_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int64]
        L.tq_packed_bytes.restype = c_size_t
        L.tq_status_string.argtypes = [c_int]
        L.tq_status_string.restype = ctypes.c_char_p
        L.tq_quantize_kv.argtypes = [POINTER(tq_quantizer), c_int, c_int, c_void_p, c_int64, c_int64,
                                     c_void_p, c_void_p, c_void_p, c_void_p]
        L.tq_quantize_kv.restype = c_int
        L.tq_append_kv.argtypes = [POINTER(tq_quantizer), c_int, c_int, c_void_p, c_int64, c_int64, c_void_p,
                                   c_int64, c_void_p, c_void_p, c_void_p, c_void_p]
        L.tq_append_kv.restype = c_int
        L.tq_append_kv_pair.argtypes = [POINTER(tq_quantizer), POINTER(tq_quantizer), c_int, c_void_p, c_void_p,
                                        c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p]
        L.tq_append_kv_pair.restype = c_int
        L.tq_kv_bit_allocation.argtypes = [c_double, c_double, POINTER(c_int), POINTER(c_int)]
        L.tq_kv_bit_allocation.restype = c_int
        L.tq_decode_paged_workspace_bytes.argtypes = [POINTER(tq_kv_desc), POINTER(tq_kv_desc), c_int, c_int, c_int,
                                                      c_int, c_int]
        L.tq_decode_paged_workspace_bytes.restype = c_size_t
        L.tq_decode_attn_paged.argtypes = [POINTER(tq_kv_desc), POINTER(tq_kv_desc), c_void_p, c_int, c_int, c_int,
                                           c_int, c_int, c_void_p, c_void_p, c_int, c_int, c_int64, c_float,
                                           c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.tq_decode_attn_paged.restype = c_int
        L.tq_decode_workspace_bytes.argtypes = [POINTER(tq_kv_desc), POINTER(tq_kv_desc), c_int, c_int, c_int, c_int]
        L.tq_decode_workspace_bytes.restype = c_size_t
        L.tq_decode_attn.argtypes = [POINTER(tq_kv_desc), POINTER(tq_kv_desc), c_void_p, c_int, c_int, c_int, c_int,
                                     c_int, c_void_p, c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.tq_decode_attn.restype = c_int
        L.tq_decode_attn_noalloc.argtypes = [POINTER(tq_kv_desc), POINTER(tq_kv_desc), c_void_p, c_int, c_int, c_int,
                                             c_int, c_int, c_void_p, c_float, c_void_p, c_void_p, c_void_p]
        L.tq_decode_attn_noalloc.restype = c_int
        L.tq_decode_step.argtypes = [POINTER(tq_kv_desc), POINTER(tq_kv_desc), c_void_p, c_void_p, c_int, c_void_p,
                                     c_int, c_int, c_int, c_int, c_int, c_void_p, c_float, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]
        L.tq_decode_step.restype = c_int
        L.tq_search_workspace_bytes.argtypes = [POINTER(tq_group), c_int64, c_int, c_int]
        L.tq_search_workspace_bytes.restype = c_size_t
        L.tq_search_topk.argtypes = [POINTER(tq_group), c_int64, c_void_p, c_int, c_int, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]
        L.tq_search_topk.restype = c_int
        L.tq_fold_bytes.argtypes = [c_int]
        L.tq_fold_bytes.restype = c_size_t
        L.tq_fold_qjl.argtypes = [POINTER(tq_quantizer), c_void_p, c_void_p]
        L.tq_fold_qjl.restype = c_int
        _lib = L
    return _lib


def _ptr(x) -> int | None:
    """Device (or host) address of a tensor, or the integer / None given."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _check(rc: int, where: str) -> None:
    if rc != TQ_OK:
        raise TQError(rc, where)


def tq_status_string(status: int) -> str:
    return lib().tq_status_string(status).decode()


def tq_build_codebook(d: int, mse_bits: int, max_iter: int = 0):
    """Returns (centroids, thresholds, D) as Python lists / float (host, fp64)."""
    L = 1 << mse_bits
    c = (c_double * L)()
    t = (c_double * max(L - 1, 1))()
    D = c_double()
    _check(lib().tq_build_codebook(d, mse_bits, c, t, ctypes.byref(D), max_iter), "tq_build_codebook")
    return list(c), list(t)[: L - 1], D.value


def tq_quantizer_init(d: int, mse_bits: int, variant: int, R, S=None) -> tq_quantizer:
    q = tq_quantizer()
    _check(lib().tq_quantizer_init(ctypes.byref(q), d, mse_bits, variant, _ptr(R), _ptr(S)), "tq_quantizer_init")
    return q


def tq_fold_bytes(d: int) -> int:
    return int(lib().tq_fold_bytes(d))


def tq_fold_qjl(q: tq_quantizer, SR, stream=None) -> None:
    """Fill SR (tq_fold_bytes(q.d) bytes) with S R and its largest row norm;
    assign q.SR = SR's address to use it (see tq_quantizer_fold)."""
    _check(lib().tq_fold_qjl(ctypes.byref(q), _ptr(SR), _stream(stream)), "tq_fold_qjl")


def tq_quantizer_fold(q: tq_quantizer, SR, stream=None) -> tq_quantizer:
    """tq_fold_qjl into SR, then return q with q.SR pointing at it."""
    tq_fold_qjl(q, SR, stream)
    q.SR = _ptr(SR)
    return q


def tq_packed_bytes(d: int, mse_bits: int, variant: int, layout: int, n: int) -> int:
    return int(lib().tq_packed_bytes(d, mse_bits, variant, layout, n))


def tq_quantize_kv(q: tq_quantizer, layout: int, in_dtype: int, x, n: int, x_stride_elems: int,
                   packed, norm, rnorm=None, stream=None) -> None:
    _check(lib().tq_quantize_kv(ctypes.byref(q), layout, in_dtype, _ptr(x), n, x_stride_elems, _ptr(packed),
                                _ptr(norm), _ptr(rnorm), _stream(stream)), "tq_quantize_kv")


def tq_append_kv(q: tq_quantizer, layout: int, in_dtype: int, x, n: int, x_stride_elems: int, rows,
                 cache_rows: int, packed, norm, rnorm=None, stream=None) -> None:
    _check(lib().tq_append_kv(ctypes.byref(q), layout, in_dtype, _ptr(x), n, x_stride_elems, _ptr(rows),
                              cache_rows, _ptr(packed), _ptr(norm), _ptr(rnorm), _stream(stream)), "tq_append_kv")


def tq_append_kv_pair(qk: tq_quantizer, qv: tq_quantizer, in_dtype: int, xk, xv, n: int, xk_stride_elems: int,
                      xv_stride_elems: int, rows, cache_rows: int, kpacked, knorm, krnorm, vpacked, vnorm,
                      vrnorm=None, stream=None) -> None:
    _check(lib().tq_append_kv_pair(ctypes.byref(qk), ctypes.byref(qv), in_dtype, _ptr(xk), _ptr(xv), n,
                                   xk_stride_elems, xv_stride_elems, _ptr(rows), cache_rows, _ptr(kpacked),
                                   _ptr(knorm), _ptr(krnorm), _ptr(vpacked), _ptr(vnorm), _ptr(vrnorm),
                                   _stream(stream)), "tq_append_kv_pair")


def tq_kv_bit_allocation(key_norm: float, value_norm: float) -> tuple[int, int, int]:
    """(class, key_bits, value_bits) for typical key and value norms."""
    kb, vb = c_int(0), c_int(0)
    rc = lib().tq_kv_bit_allocation(float(key_norm), float(value_norm), ctypes.byref(kb), ctypes.byref(vb))
    _check(min(rc, 0), "tq_kv_bit_allocation")
    return rc, kb.value, vb.value


def make_group(q: tq_quantizer, ch_offset: int, packed, norm, rnorm, seq_stride: int) -> tq_group:
    g = tq_group()
    g.q = q
    g.ch_offset = ch_offset
    g.packed = _ptr(packed)
    g.norm = _ptr(norm)
    g.rnorm = _ptr(rnorm)
    g.seq_stride = seq_stride
    return g


def make_desc(groups) -> tq_kv_desc:
    dsc = tq_kv_desc()
    dsc.n_groups = len(groups)
    for i, g in enumerate(groups):
        dsc.g[i] = g
    return dsc


def tq_decode_workspace_bytes(k: tq_kv_desc, v: tq_kv_desc, B: int, Hq: int, Hkv: int, T_max: int) -> int:
    return int(lib().tq_decode_workspace_bytes(ctypes.byref(k), ctypes.byref(v), B, Hq, Hkv, T_max))


def tq_decode_attn(k: tq_kv_desc, v: tq_kv_desc, q, q_dtype: int, B: int, Hq: int, Hkv: int, T_max: int,
                   seq_lens, scale: float, out, scores_out, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().tq_decode_attn(ctypes.byref(k), ctypes.byref(v), _ptr(q), q_dtype, B, Hq, Hkv, T_max,
                                _ptr(seq_lens), scale, _ptr(out), _ptr(scores_out), _ptr(ws), ws_bytes,
                                _stream(stream)), "tq_decode_attn")


def tq_decode_attn_noalloc(k: tq_kv_desc, v: tq_kv_desc, q, q_dtype: int, B: int, Hq: int, Hkv: int, T_max: int,
                           seq_lens, scale: float, out, scores_out, stream=None) -> None:
    _check(lib().tq_decode_attn_noalloc(ctypes.byref(k), ctypes.byref(v), _ptr(q), q_dtype, B, Hq, Hkv, T_max,
                                        _ptr(seq_lens), scale, _ptr(out), _ptr(scores_out), _stream(stream)),
           "tq_decode_attn_noalloc")


def tq_decode_step(k: tq_kv_desc, v: tq_kv_desc, k_new, v_new, kv_dtype: int, q, q_dtype: int, B: int, Hq: int,
                   Hkv: int, T_max: int, seq_lens, scale: float, out, scores_out, ws, ws_bytes: int,
                   stream=None) -> None:
    _check(lib().tq_decode_step(ctypes.byref(k), ctypes.byref(v), _ptr(k_new), _ptr(v_new), kv_dtype, _ptr(q),
                                q_dtype, B, Hq, Hkv, T_max, _ptr(seq_lens), scale, _ptr(out), _ptr(scores_out),
                                _ptr(ws), ws_bytes, _stream(stream)), "tq_decode_step")


def tq_decode_paged_workspace_bytes(k: tq_kv_desc, v: tq_kv_desc, B: int, Hq: int, Hkv: int, T_max: int,
                                    block_tokens: int) -> int:
    return int(lib().tq_decode_paged_workspace_bytes(ctypes.byref(k), ctypes.byref(v), B, Hq, Hkv, T_max,
                                                     block_tokens))


def tq_decode_attn_paged(k: tq_kv_desc, v: tq_kv_desc, q, q_dtype: int, B: int, Hq: int, Hkv: int, T_max: int,
                         seq_lens, block_table, max_blocks: int, block_tokens: int, num_blocks: int, scale: float,
                         out, scores_out, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().tq_decode_attn_paged(ctypes.byref(k), ctypes.byref(v), _ptr(q), q_dtype, B, Hq, Hkv, T_max,
                                      _ptr(seq_lens), _ptr(block_table), max_blocks, block_tokens, num_blocks,
                                      scale, _ptr(out), _ptr(scores_out), _ptr(ws), ws_bytes, _stream(stream)),
           "tq_decode_attn_paged")


def tq_search_workspace_bytes(db: tq_group, N: int, Q: int, k: int) -> int:
    return int(lib().tq_search_workspace_bytes(ctypes.byref(db), N, Q, k))


def tq_search_topk(db: tq_group, N: int, queries, Q: int, k: int, out_idx, out_score, ws, ws_bytes: int,
                   stream=None) -> None:
    _check(lib().tq_search_topk(ctypes.byref(db), N, _ptr(queries), Q, k, _ptr(out_idx), _ptr(out_score),
                                _ptr(ws), ws_bytes, _stream(stream)), "tq_search_topk")
