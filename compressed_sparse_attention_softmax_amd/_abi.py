"""Thin ctypes binding of libcsa (include/csa.h): argument marshalling only.

Each function has the name of the C entry point it calls.  Tensors are torch
tensors on the GPU; the binding checks dtype, device, contiguity and shapes,
passes ``data_ptr()`` and the current HIP stream, and raises ``CSAError``
with ``csa_last_error()`` on a non-zero status.  Every step of the path runs
in the library's kernels; nothing here computes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

CSA_F32, CSA_BF16 = 0, 1
STATUS = {0: "CSA_OK", -1: "CSA_ERR_ARG", -2: "CSA_ERR_SHAPE", -3: "CSA_ERR_DTYPE",
          -4: "CSA_ERR_UNSUPPORTED", -5: "CSA_ERR_WORKSPACE", -6: "CSA_ERR_HIP"}

# every symbol include/csa.h declares
EXPORTS = ["csa_compress", "csa_compress_bwd_workspace", "csa_compress_bwd", "csa_index_topk_workspace", "csa_index_topk",
           "csa_compress_strided", "csa_compress_bwd_strided", "csa_index_topk_strided",
           "csa_sparse_attn_fwd", "csa_sparse_attn_bwd_workspace", "csa_sparse_attn_bwd_query_block",
           "csa_sparse_attn_bwd", "csa_sparse_attn_bwd_noalloc", "csa_sparse_attn_fwd_strided",
           "csa_sparse_attn_bwd_strided", "csa_indexer_loss_workspace", "csa_indexer_loss", "csa_indexer_loss_dense_workspace",
           "csa_indexer_loss_dense", "csa_dsa_gqa_workspace", "csa_dsa_gqa_fwd",
           "csa_dsa_gqa_bwd", "csa_last_error", "csa_version", "csa_timing_enable", "csa_timing_read", "csa_kernel_name"]

# kernel ids of the timing hook (enum csa_kernel_id)
CSA_K_COMPRESS_FWD, CSA_K_COMPRESS_BWD, CSA_K_INDEX_TOPK, CSA_K_ATTN_FWD = 0, 1, 2, 3
CSA_K_ATTN_DQ, CSA_K_ATTN_ROWS, CSA_K_ATTN_REDUCE = 4, 5, 6
CSA_K_LOSS_QUERY, CSA_K_LOSS_KEYS, CSA_K_LOSS_REDUCE = 7, 8, 9
CSA_K_COMPRESS_EPI = 10


class CSAError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(code, code)}: {msg}")
        self.code = code


class csa_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("b", "sq", "h", "d", "ratio", "span", "window", "idx_heads", "idx_dim", "topk")]


class csa_attn_strides(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("q_b", "q_s", "q_h", "kv_b", "kv_s", "lse_b", "lse_s")]


class csa_compress_strides(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("x_b", "x_s", "z_b", "z_s")]


class csa_index_strides(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("qi_b", "qi_s", "qi_h", "ki_b", "ki_s", "w_b", "w_s")]


class csa_gqa_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("b", "sq", "h", "h_kv", "d_qk", "d_v", "topk")]


_lib = None


def load(path: Optional[str] = None):
    """Load libcsa.so (built in-tree).  Raises if it is missing: there is no
    fallback implementation."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libcsa.so not found at {p}; build it with "
                           "`python -m compressed_sparse_attention_softmax_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(csa_dims)
    lib.csa_compress.argtypes = [D, i, vp, vp, i, vp, f, i, f, vp, vp, vp]
    lib.csa_compress_bwd_workspace.argtypes = [D]
    lib.csa_compress_bwd_workspace.restype = sz
    lib.csa_compress_bwd.argtypes = [D, i, vp, vp, i, vp, f, i, f, vp, vp, vp, vp, vp, sz, vp]
    lib.csa_index_topk_workspace.argtypes = [D]
    lib.csa_index_topk_workspace.restype = sz
    lib.csa_index_topk.argtypes = [D, i, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.csa_sparse_attn_fwd.argtypes = [D, i, vp, vp, vp, vp, vp, vp, f, vp, vp, vp]
    lib.csa_sparse_attn_bwd_workspace.argtypes = [D]
    lib.csa_sparse_attn_bwd_workspace.restype = sz
    lib.csa_sparse_attn_bwd_query_block.argtypes = [D, i]
    lib.csa_sparse_attn_bwd_query_block.restype = i
    lib.csa_sparse_attn_bwd.argtypes = [D, i, vp, vp, vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.csa_sparse_attn_bwd_noalloc.argtypes = [D, i, vp, vp, vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, vp, vp]
    ST = ctypes.POINTER(csa_attn_strides)
    lib.csa_sparse_attn_fwd_strided.argtypes = [D, ST, i, vp, vp, vp, vp, vp, vp, f, vp, vp, vp]
    lib.csa_sparse_attn_bwd_strided.argtypes = [D, ST, i, vp, vp, vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, vp, vp,
                                                sz, vp]
    CST = ctypes.POINTER(csa_compress_strides)
    lib.csa_compress_strided.argtypes = [D, CST, i, vp, vp, i, vp, f, i, f, vp, vp, vp]
    lib.csa_compress_bwd_strided.argtypes = [D, CST, i, vp, vp, i, vp, f, i, f, vp, vp, vp, vp, vp, sz, vp]
    lib.csa_index_topk_strided.argtypes = [D, ctypes.POINTER(csa_index_strides), i, vp, vp, vp, vp, vp, vp, vp, sz,
                                           vp]
    lib.csa_indexer_loss_workspace.argtypes = [D]
    lib.csa_indexer_loss_workspace.restype = sz
    lib.csa_indexer_loss.argtypes = [D, i, vp, vp, vp, vp, vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.csa_indexer_loss_dense_workspace.argtypes = [D, sz]
    lib.csa_indexer_loss_dense_workspace.restype = sz
    lib.csa_indexer_loss_dense.argtypes = [D, i, vp, vp, vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, sz, vp]
    GD = ctypes.POINTER(csa_gqa_dims)
    lib.csa_dsa_gqa_workspace.argtypes = [GD, i, i]
    lib.csa_dsa_gqa_workspace.restype = sz
    lib.csa_dsa_gqa_fwd.argtypes = [GD, i, vp, vp, vp, vp, f, vp, vp, vp, sz, vp]
    lib.csa_dsa_gqa_bwd.argtypes = [GD, i, vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.csa_last_error.argtypes = []
    lib.csa_last_error.restype = ctypes.c_char_p
    lib.csa_version.argtypes = []
    lib.csa_timing_enable.argtypes = [i]
    lib.csa_timing_read.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]
    lib.csa_kernel_name.argtypes = [i]
    lib.csa_kernel_name.restype = ctypes.c_char_p
    for fn in ("csa_compress", "csa_compress_bwd", "csa_index_topk", "csa_compress_strided", "csa_compress_bwd_strided",
               "csa_index_topk_strided", "csa_sparse_attn_fwd",
               "csa_sparse_attn_bwd", "csa_sparse_attn_bwd_noalloc", "csa_sparse_attn_fwd_strided",
               "csa_sparse_attn_bwd_strided", "csa_indexer_loss", "csa_indexer_loss_dense", "csa_dsa_gqa_fwd", "csa_dsa_gqa_bwd", "csa_version", "csa_timing_enable", "csa_timing_read"):
        getattr(lib, fn).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def make_dims(b, sq, h=1, d=64, ratio=1, span=1, window=1, idx_heads=1, idx_dim=32, topk=0) -> csa_dims:
    return csa_dims(b, sq, h, d, ratio, span, window, idx_heads, idx_dim, topk)


def dims_of(wl) -> csa_dims:
    """csa_dims of a workload description (any object with the csa_dims fields)."""
    return csa_dims(wl.b, wl.sq, wl.h, wl.d, wl.ratio, wl.span, wl.window, wl.idx_heads,
                    wl.idx_dim, wl.topk)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor], *, shape=None, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _call(fn: str, *args) -> None:
    lib = load()
    rc = getattr(lib, fn)(*args)
    if rc != 0:
        raise CSAError(fn, rc, lib.csa_last_error().decode())


def n_compressed(dims: csa_dims) -> int:
    return dims.sq // dims.ratio if dims.ratio >= 1 else 0


def kprime(dims: csa_dims) -> int:
    return min(dims.topk, n_compressed(dims))


def csa_compress(dims: csa_dims, x, z, c, c32=None, stream=None, norm_w=None, norm_eps: float = 1e-6,
                 rope_dim: int = 0, rope_base: float = 40000.0) -> None:
    dt = x.dtype
    b, S, D = dims.b, dims.sq, dims.d
    zc = z.shape[-1]
    nc = n_compressed(dims)
    _call("csa_compress", ctypes.byref(dims), _dtype_code(x),
          _ptr(x, shape=(b, S, D), dtype=dt, name="x"), _ptr(z, shape=(b, S, zc), dtype=dt, name="z"),
          zc, _ptr(norm_w, shape=(D,), dtype=torch.float32, name="norm_w"), ctypes.c_float(norm_eps),
          int(rope_dim), ctypes.c_float(rope_base), _ptr(c, shape=(b, nc, D), dtype=dt, name="c"),
          _ptr(c32, shape=(b, nc, D), dtype=torch.float32, name="c32"), _stream(stream))


def csa_compress_bwd_workspace(dims: csa_dims) -> int:
    return int(load().csa_compress_bwd_workspace(ctypes.byref(dims)))


def csa_compress_bwd(dims: csa_dims, x, z, dc, dx, dz, stream=None, norm_w=None, norm_eps: float = 1e-6,
                     rope_dim: int = 0, rope_base: float = 40000.0, dnorm_w=None, ws=None) -> None:
    dt = x.dtype
    b, S, D = dims.b, dims.sq, dims.d
    zc = z.shape[-1]
    nc = n_compressed(dims)
    f32 = torch.float32
    _call("csa_compress_bwd", ctypes.byref(dims), _dtype_code(x),
          _ptr(x, shape=(b, S, D), dtype=dt, name="x"), _ptr(z, shape=(b, S, zc), dtype=dt, name="z"),
          zc, _ptr(norm_w, shape=(D,), dtype=f32, name="norm_w"), ctypes.c_float(norm_eps), int(rope_dim),
          ctypes.c_float(rope_base), _ptr(dc, shape=(b, nc, D), dtype=f32, name="dc"),
          _ptr(dx, shape=(b, S, D), dtype=f32, name="dx"), _ptr(dz, shape=(b, S, zc), dtype=f32, name="dz"),
          _ptr(dnorm_w, shape=(D,), dtype=f32, name="dnorm_w"), _ptr(ws, name="ws"),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def csa_index_topk_workspace(dims: csa_dims) -> int:
    return int(load().csa_index_topk_workspace(ctypes.byref(dims)))


def _doc_ptr(dims, doc_ids):
    return _ptr(doc_ids, shape=(dims.b, dims.sq), dtype=torch.int32, name="doc_ids")


def csa_index_topk(dims: csa_dims, q_i, k_i, w, idx, score=None, ws=None, stream=None, doc_ids=None) -> None:
    dt = q_i.dtype
    b, S = dims.b, dims.sq
    nc, kp = n_compressed(dims), kprime(dims)
    f32 = torch.float32
    _call("csa_index_topk", ctypes.byref(dims), _dtype_code(q_i),
          _ptr(q_i, shape=(b, S, dims.idx_heads, dims.idx_dim), dtype=dt, name="q_i"),
          _ptr(k_i, shape=(b, nc, dims.idx_dim), dtype=dt, name="k_i"),
          _ptr(w, shape=(b, S, dims.idx_heads), dtype=f32, name="w"), _doc_ptr(dims, doc_ids),
          _ptr(idx, shape=(b, S, kp), dtype=torch.int32, name="idx"),
          _ptr(score, shape=(b, S, kp), dtype=f32, name="score"),
          _ptr(ws, name="ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def compress_strides_of(x, z) -> csa_compress_strides:
    """csa_compress_strides of views x [b, sq, d] and z [b, sq, z_channels]."""
    return csa_compress_strides(x.stride(0), x.stride(1), z.stride(0), z.stride(1))


def csa_compress_strided(dims: csa_dims, x, z, c, c32=None, stream=None, norm_w=None, norm_eps: float = 1e-6,
                         rope_dim: int = 0, rope_base: float = 40000.0) -> None:
    """csa_compress over views x [b, sq, d] and z [b, sq, z_channels] whose
    last axis is contiguous (c and c32 contiguous)."""
    dt = x.dtype
    b, S, D = dims.b, dims.sq, dims.d
    zc = z.shape[-1]
    nc = n_compressed(dims)
    st = compress_strides_of(x, z)
    _call("csa_compress_strided", ctypes.byref(dims), ctypes.byref(st), _dtype_code(x),
          _strided_ptr(x, (b, S, D), dt, "x"), _strided_ptr(z, (b, S, zc), dt, "z"), zc,
          _ptr(norm_w, shape=(D,), dtype=torch.float32, name="norm_w"), ctypes.c_float(norm_eps), int(rope_dim),
          ctypes.c_float(rope_base), _ptr(c, shape=(b, nc, D), dtype=dt, name="c"),
          _ptr(c32, shape=(b, nc, D), dtype=torch.float32, name="c32"), _stream(stream))


def csa_compress_bwd_strided(dims: csa_dims, x, z, dc, dx, dz, stream=None, norm_w=None, norm_eps: float = 1e-6,
                             rope_dim: int = 0, rope_base: float = 40000.0, dnorm_w=None, ws=None) -> None:
    """csa_compress_bwd over strided views: dx (fp32) shares x's element
    strides, dz shares z's; dc is contiguous."""
    dt = x.dtype
    b, S, D = dims.b, dims.sq, dims.d
    zc = z.shape[-1]
    nc = n_compressed(dims)
    f32 = torch.float32
    st = compress_strides_of(x, z)
    _call("csa_compress_bwd_strided", ctypes.byref(dims), ctypes.byref(st), _dtype_code(x),
          _strided_ptr(x, (b, S, D), dt, "x"), _strided_ptr(z, (b, S, zc), dt, "z"), zc,
          _ptr(norm_w, shape=(D,), dtype=f32, name="norm_w"), ctypes.c_float(norm_eps), int(rope_dim),
          ctypes.c_float(rope_base), _ptr(dc, shape=(b, nc, D), dtype=f32, name="dc"),
          _strided_ptr(dx, (b, S, D), f32, "dx", like=x), _strided_ptr(dz, (b, S, zc), f32, "dz", like=z),
          _ptr(dnorm_w, shape=(D,), dtype=f32, name="dnorm_w"), _ptr(ws, name="ws"),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def index_strides_of(q_i, k_i, w) -> csa_index_strides:
    """csa_index_strides of views q_i [b, sq, hi, di], k_i [b, n_c, di] and w [b, sq, hi] (w may be None)."""
    return csa_index_strides(q_i.stride(0), q_i.stride(1), q_i.stride(2), k_i.stride(0), k_i.stride(1),
                             w.stride(0) if w is not None else 0, w.stride(1) if w is not None else 0)


def csa_index_topk_strided(dims: csa_dims, q_i, k_i, w, idx, score=None, ws=None, stream=None, doc_ids=None) -> None:
    """csa_index_topk over views q_i, k_i and w whose last axis is contiguous
    (idx, score and doc_ids contiguous)."""
    dt = q_i.dtype
    b, S = dims.b, dims.sq
    nc, kp = n_compressed(dims), kprime(dims)
    f32 = torch.float32
    st = index_strides_of(q_i, k_i, w)
    _call("csa_index_topk_strided", ctypes.byref(dims), ctypes.byref(st), _dtype_code(q_i),
          _strided_ptr(q_i, (b, S, dims.idx_heads, dims.idx_dim), dt, "q_i"),
          _strided_ptr(k_i, (b, nc, dims.idx_dim), dt, "k_i"),
          _strided_ptr(w, (b, S, dims.idx_heads), f32, "w"), _doc_ptr(dims, doc_ids),
          _ptr(idx, shape=(b, S, kp), dtype=torch.int32, name="idx"),
          _ptr(score, shape=(b, S, kp), dtype=f32, name="score"),
          _ptr(ws, name="ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def _attn_ptrs(dims, q, kv, c, idx, sink, doc_ids):
    dt = q.dtype
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    nc = n_compressed(dims) if c is not None else 0
    if sink is not None and sink.numel() != H:
        raise CSAError("csa_sparse_attn", -2, f"sink has {sink.numel()} entries, h = {H}")
    return (_ptr(q, shape=(b, S, H, D), dtype=dt, name="q"), _ptr(kv, shape=(b, S, D), dtype=dt, name="kv"),
            _ptr(c, shape=(b, nc, D), dtype=dt, name="c"),
            _ptr(idx, shape=(b, S, kprime(dims)), dtype=torch.int32, name="idx"), _doc_ptr(dims, doc_ids),
            _ptr(sink, shape=(H,), dtype=torch.float32, name="sink"))


def csa_sparse_attn_fwd(dims: csa_dims, q, kv, c, idx, sink, scale: float, out, lse, stream=None,
                        doc_ids=None) -> None:
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    _call("csa_sparse_attn_fwd", ctypes.byref(dims), _dtype_code(q),
          *_attn_ptrs(dims, q, kv, c, idx, sink, doc_ids),
          ctypes.c_float(scale), _ptr(out, shape=(b, S, H, D), dtype=q.dtype, name="out"),
          _ptr(lse, shape=(b, S, H), dtype=torch.float32, name="lse"), _stream(stream))


def csa_sparse_attn_bwd_workspace(dims: csa_dims) -> int:
    return int(load().csa_sparse_attn_bwd_workspace(ctypes.byref(dims)))


def csa_sparse_attn_bwd_query_block(dims: csa_dims, with_compressed: bool = True) -> int:
    return int(load().csa_sparse_attn_bwd_query_block(ctypes.byref(dims), int(bool(with_compressed))))


def csa_sparse_attn_bwd(dims: csa_dims, q, kv, c, idx, sink, scale: float, out, lse, dout, dq, dkv, dc,
                        dsink=None, ws=None, stream=None, doc_ids=None) -> None:
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    f32 = torch.float32
    nc = n_compressed(dims) if c is not None else 0
    _call("csa_sparse_attn_bwd", ctypes.byref(dims), _dtype_code(q),
          *_attn_ptrs(dims, q, kv, c, idx, sink, doc_ids),
          ctypes.c_float(scale), _ptr(out, shape=(b, S, H, D), dtype=q.dtype, name="out"),
          _ptr(lse, shape=(b, S, H), dtype=f32, name="lse"),
          _ptr(dout, shape=(b, S, H, D), dtype=q.dtype, name="dout"),
          _ptr(dq, shape=(b, S, H, D), dtype=q.dtype, name="dq"),
          _ptr(dkv, shape=(b, S, D), dtype=f32, name="dkv"), _ptr(dc, shape=(b, nc, D), dtype=f32, name="dc"),
          _ptr(dsink, shape=(H,), dtype=f32, name="dsink"), _ptr(ws, name="ws"),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def csa_sparse_attn_bwd_noalloc(dims: csa_dims, q, kv, c, idx, sink, scale: float, out, lse, dout, dq, dkv, dc,
                                dsink=None, stream=None, doc_ids=None) -> None:
    """csa_sparse_attn_bwd with the library's fixed device scratch instead of a
    caller workspace (for callers that cannot allocate)."""
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    f32 = torch.float32
    nc = n_compressed(dims) if c is not None else 0
    _call("csa_sparse_attn_bwd_noalloc", ctypes.byref(dims), _dtype_code(q),
          *_attn_ptrs(dims, q, kv, c, idx, sink, doc_ids),
          ctypes.c_float(scale), _ptr(out, shape=(b, S, H, D), dtype=q.dtype, name="out"),
          _ptr(lse, shape=(b, S, H), dtype=f32, name="lse"),
          _ptr(dout, shape=(b, S, H, D), dtype=q.dtype, name="dout"),
          _ptr(dq, shape=(b, S, H, D), dtype=q.dtype, name="dq"),
          _ptr(dkv, shape=(b, S, D), dtype=f32, name="dkv"), _ptr(dc, shape=(b, nc, D), dtype=f32, name="dc"),
          _ptr(dsink, shape=(H,), dtype=f32, name="dsink"), _stream(stream))


def _strided_ptr(t, shape, dtype, name, like=None):
    """Pointer of a view of logical shape `shape` whose last axis is contiguous;
    with `like` (a tensor of the same family) its strides must match on every
    axis of extent > 1."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous along its last axis")
    if like is not None:
        for ax, n in enumerate(shape[:-1]):
            if n > 1 and t.stride(ax) != like.stride(ax):
                raise ValueError(f"{name} strides {t.stride()} differ from {like.stride()}")
    return ctypes.c_void_p(t.data_ptr())


def attn_strides_of(q, kv, lse) -> csa_attn_strides:
    """csa_attn_strides of views q [b, sq, h, d], kv [b, sq, d] and lse [b, sq, h]."""
    return csa_attn_strides(q.stride(0), q.stride(1), q.stride(2), kv.stride(0), kv.stride(1), lse.stride(0),
                            lse.stride(1))


def _strided_attn_ptrs(dims, q, kv, c, idx, sink, doc_ids):
    dt = q.dtype
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    nc = n_compressed(dims) if c is not None else 0
    if sink is not None and sink.numel() != H:
        raise CSAError("csa_sparse_attn", -2, f"sink has {sink.numel()} entries, h = {H}")
    return (_strided_ptr(q, (b, S, H, D), dt, "q"), _strided_ptr(kv, (b, S, D), dt, "kv"),
            _ptr(c, shape=(b, nc, D), dtype=dt, name="c"),
            _ptr(idx, shape=(b, S, kprime(dims)), dtype=torch.int32, name="idx"), _doc_ptr(dims, doc_ids),
            _ptr(sink, shape=(H,), dtype=torch.float32, name="sink"))


def csa_sparse_attn_fwd_strided(dims: csa_dims, q, kv, c, idx, sink, scale: float, out, lse, stream=None,
                                doc_ids=None) -> None:
    """csa_sparse_attn_fwd over strided views (e.g. sequence-major tensors
    viewed as [b, sq, ...]); out shares q's strides.  c, idx, doc_ids and sink
    stay contiguous."""
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    st = attn_strides_of(q, kv, lse)
    _call("csa_sparse_attn_fwd_strided", ctypes.byref(dims), ctypes.byref(st), _dtype_code(q),
          *_strided_attn_ptrs(dims, q, kv, c, idx, sink, doc_ids), ctypes.c_float(scale),
          _strided_ptr(out, (b, S, H, D), q.dtype, "out", like=q),
          _strided_ptr(lse, (b, S, H), torch.float32, "lse"), _stream(stream))


def csa_sparse_attn_bwd_strided(dims: csa_dims, q, kv, c, idx, sink, scale: float, out, lse, dout, dq, dkv, dc,
                                dsink=None, ws=None, stream=None, doc_ids=None) -> None:
    """csa_sparse_attn_bwd over strided views: out, dout and dq share q's
    strides, dkv (fp32) shares kv's element strides."""
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    f32 = torch.float32
    nc = n_compressed(dims) if c is not None else 0
    st = attn_strides_of(q, kv, lse)
    _call("csa_sparse_attn_bwd_strided", ctypes.byref(dims), ctypes.byref(st), _dtype_code(q),
          *_strided_attn_ptrs(dims, q, kv, c, idx, sink, doc_ids), ctypes.c_float(scale),
          _strided_ptr(out, (b, S, H, D), q.dtype, "out", like=q),
          _strided_ptr(lse, (b, S, H), f32, "lse"),
          _strided_ptr(dout, (b, S, H, D), q.dtype, "dout", like=q),
          _strided_ptr(dq, (b, S, H, D), q.dtype, "dq", like=q),
          _strided_ptr(dkv, (b, S, D), f32, "dkv", like=kv), _ptr(dc, shape=(b, nc, D), dtype=f32, name="dc"),
          _ptr(dsink, shape=(H,), dtype=f32, name="dsink"), _ptr(ws, name="ws"),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def csa_indexer_loss_workspace(dims: csa_dims) -> int:
    return int(load().csa_indexer_loss_workspace(ctypes.byref(dims)))


def csa_indexer_loss(dims: csa_dims, q, c, lse, q_i, k_i, w, idx, score, scale: float, kl=None, dkl=None,
                     dq_i=None, dw=None, dk_i=None, ws=None, stream=None) -> None:
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    HI, DI = dims.idx_heads, dims.idx_dim
    nc, kp = n_compressed(dims), kprime(dims)
    dt, f32 = q.dtype, torch.float32
    _call("csa_indexer_loss", ctypes.byref(dims), _dtype_code(q),
          _ptr(q, shape=(b, S, H, D), dtype=dt, name="q"), _ptr(c, shape=(b, nc, D), dtype=dt, name="c"),
          _ptr(lse, shape=(b, S, H), dtype=f32, name="lse"),
          _ptr(q_i, shape=(b, S, HI, DI), dtype=dt, name="q_i"), _ptr(k_i, shape=(b, nc, DI), dtype=dt, name="k_i"),
          _ptr(w, shape=(b, S, HI), dtype=f32, name="w"),
          _ptr(idx, shape=(b, S, kp), dtype=torch.int32, name="idx"),
          _ptr(score, shape=(b, S, kp), dtype=f32, name="score"), ctypes.c_float(scale),
          _ptr(dkl, shape=(b, S), dtype=f32, name="dkl"), _ptr(kl, shape=(b, S), dtype=f32, name="kl"),
          _ptr(dq_i, shape=(b, S, HI, DI), dtype=dt, name="dq_i"), _ptr(dw, shape=(b, S, HI), dtype=f32, name="dw"),
          _ptr(dk_i, shape=(b, nc, DI), dtype=f32, name="dk_i"), _ptr(ws, name="ws"),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def csa_indexer_loss_dense_workspace(dims: csa_dims, budget: int = 0) -> int:
    """Bytes the dense warm-up loss's plan uses within ``budget`` (at least its minimum)."""
    return int(load().csa_indexer_loss_dense_workspace(ctypes.byref(dims), int(budget)))


def csa_indexer_loss_dense(dims: csa_dims, q, c, lse, q_i, k_i, w, scale: float, kl=None, dkl=None, dq_i=None,
                           dw=None, dk_i=None, ws=None, stream=None) -> None:
    """Dense warm-up form of the indexer loss: every valid block is the support."""
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    HI, DI = dims.idx_heads, dims.idx_dim
    nc = n_compressed(dims)
    dt, f32 = q.dtype, torch.float32
    _call("csa_indexer_loss_dense", ctypes.byref(dims), _dtype_code(q),
          _ptr(q, shape=(b, S, H, D), dtype=dt, name="q"), _ptr(c, shape=(b, nc, D), dtype=dt, name="c"),
          _ptr(lse, shape=(b, S, H), dtype=f32, name="lse"),
          _ptr(q_i, shape=(b, S, HI, DI), dtype=dt, name="q_i"), _ptr(k_i, shape=(b, nc, DI), dtype=dt, name="k_i"),
          _ptr(w, shape=(b, S, HI), dtype=f32, name="w"), ctypes.c_float(scale),
          _ptr(dkl, shape=(b, S), dtype=f32, name="dkl"), _ptr(kl, shape=(b, S), dtype=f32, name="kl"),
          _ptr(dq_i, shape=(b, S, HI, DI), dtype=dt, name="dq_i"), _ptr(dw, shape=(b, S, HI), dtype=f32, name="dw"),
          _ptr(dk_i, shape=(b, nc, DI), dtype=f32, name="dk_i"), _ptr(ws, name="ws"),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def csa_dsa_gqa_workspace(g: csa_gqa_dims, dtype: torch.dtype, backward: bool) -> int:
    code = CSA_BF16 if dtype == torch.bfloat16 else CSA_F32
    return int(load().csa_dsa_gqa_workspace(ctypes.byref(g), code, int(backward)))


def _gqa_shapes(g: csa_gqa_dims):
    b, S = g.b, g.sq
    return dict(q=(b, S, g.h, g.d_qk), k=(b, S, g.h_kv, g.d_qk), v=(b, S, g.h_kv, g.d_v), out=(b, S, g.h, g.d_v),
                lse=(b, S, g.h), idx=(b, S, min(g.topk, g.sq)))


def csa_dsa_gqa_fwd(g: csa_gqa_dims, q, k, v, idx, scale: float, out, lse, ws, stream=None) -> None:
    sh, dt = _gqa_shapes(g), q.dtype
    _call("csa_dsa_gqa_fwd", ctypes.byref(g), _dtype_code(q), _ptr(q, shape=sh["q"], dtype=dt, name="q"),
          _ptr(k, shape=sh["k"], dtype=dt, name="k"), _ptr(v, shape=sh["v"], dtype=dt, name="v"),
          _ptr(idx, shape=sh["idx"], dtype=torch.int32, name="idx"), ctypes.c_float(scale),
          _ptr(out, shape=sh["out"], dtype=dt, name="out"), _ptr(lse, shape=sh["lse"], dtype=torch.float32, name="lse"),
          _ptr(ws, name="ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def csa_dsa_gqa_bwd(g: csa_gqa_dims, q, k, v, idx, scale: float, out, lse, dout, dq, dk, dv, ws,
                    stream=None) -> None:
    sh, dt, f32 = _gqa_shapes(g), q.dtype, torch.float32
    _call("csa_dsa_gqa_bwd", ctypes.byref(g), _dtype_code(q), _ptr(q, shape=sh["q"], dtype=dt, name="q"),
          _ptr(k, shape=sh["k"], dtype=dt, name="k"), _ptr(v, shape=sh["v"], dtype=dt, name="v"),
          _ptr(idx, shape=sh["idx"], dtype=torch.int32, name="idx"), ctypes.c_float(scale),
          _ptr(out, shape=sh["out"], dtype=dt, name="out"), _ptr(lse, shape=sh["lse"], dtype=f32, name="lse"),
          _ptr(dout, shape=sh["out"], dtype=dt, name="dout"), _ptr(dq, shape=sh["q"], dtype=dt, name="dq"),
          _ptr(dk, shape=sh["k"], dtype=f32, name="dk"), _ptr(dv, shape=sh["v"], dtype=f32, name="dv"),
          _ptr(ws, name="ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def csa_last_error() -> str:
    return load().csa_last_error().decode()


def csa_version() -> int:
    return int(load().csa_version())


def csa_timing_enable(kernel: int) -> None:
    """Bracket every later launch of kernel ``kernel`` (a CSA_K_* id) with HIP
    events on its stream; -1 switches timing off."""
    _call("csa_timing_enable", int(kernel))


def csa_timing_read():
    """(launches, total_ms) of the launches timed since the last read."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _call("csa_timing_read", ctypes.byref(n), ctypes.byref(ms))
    return n.value, ms.value


def csa_kernel_name(kernel: int) -> str:
    return load().csa_kernel_name(int(kernel)).decode()
