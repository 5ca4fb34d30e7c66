"""fp64 CPU oracle for the compressed sparse attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library and its Python binding never import, link or call it, and it shares
no code with them.

Two independent formulations live here:

* ``csa_oracle.c`` (loaded through ctypes, wrapped below): the plain
  definitions, one loop nest per step, over explicit candidate lists.
* ``brute.py``: a NumPy dense formulation over the unified key axis (raw rows
  followed by compressed rows) plus a sink column, used on tiny inputs to
  cross-check the C oracle.
* ``epilogue.py``: the compressor's epilogue (post-pool RMS norm and the
  rotary embedding of the compressed positions) and its backward.
* ``dsa_gqa.py``: the simplified DSA over grouped-query attention (attention
  over the keys a one-head, unit-weight indexer selected at full resolution).
* ``indexer_loss.py``: the indexer's training path (teacher target from the
  attention LSE, the student's selected scores, the KL loss and its
  gradients), plain NumPy one query row at a time.

All arrays handed to the C oracle are float64 (int32 for index lists).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_LIB = os.path.join(_HERE, "libcsa_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (plain -O2, IEEE semantics, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            i64, dp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
            lib.csa_oracle_compress.argtypes = [i64] * 6 + [dp] * 3
            lib.csa_oracle_compress_bwd.argtypes = [i64] * 6 + [dp] * 5
            lib.csa_oracle_index_scores.argtypes = [i64] * 4 + [dp] * 3 + [i64, ip, ip, i64, ip, dp]
            lib.csa_oracle_topk.argtypes = [i64] * 4 + [ip, ip, i64, ip, dp, ip, dp]
            lib.csa_oracle_attn_fwd.argtypes = ([i64] * 7 + [dp] * 3 + [ip, dp, ctypes.c_double,
                                                 i64, ip, ip, ip, dp, dp])
            lib.csa_oracle_attn_bwd.argtypes = ([i64] * 7 + [dp] * 3 + [ip, dp, ctypes.c_double,
                                                 i64, ip, ip, ip, dp, dp, dp, dp, dp])
            for f in (lib.csa_oracle_compress, lib.csa_oracle_compress_bwd,
                      lib.csa_oracle_index_scores, lib.csa_oracle_topk,
                      lib.csa_oracle_attn_fwd, lib.csa_oracle_attn_bwd):
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _doc(doc):
    """doc_ids [b, S] as contiguous int32 (or None) and the row length S."""
    if doc is None:
        return None, 0
    d = np.ascontiguousarray(np.asarray(doc, dtype=np.int32))
    return d, d.shape[1]


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed ({rc})")


def _rows(rows, b, sq):
    """rows: None (all rows) or an int array [n, 2] of (batch, t)."""
    if rows is None:
        bb, tt = np.meshgrid(np.arange(b), np.arange(sq), indexing="ij")
        rows = np.stack([bb.ravel(), tt.ravel()], axis=1)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return rows, np.ascontiguousarray(rows[:, 0]), np.ascontiguousarray(rows[:, 1])


def compress(x, z, ratio, span):
    """x [b,S,D], z [b,S,zc] -> C [b,S//ratio,D] in fp64."""
    x, z = _f64(x), _f64(z)
    b, S, D = x.shape
    zc = z.shape[2]
    out = np.zeros((b, S // ratio, D))
    _check(_load().csa_oracle_compress(b, S, D, ratio, span, zc, _ptr(x), _ptr(z), _ptr(out)),
           "compress")
    return out


def compress_bwd(x, z, dc, ratio, span):
    """-> (dX [b,S,D], dZ [b,S,zc]) in fp64."""
    x, z, dc = _f64(x), _f64(z), _f64(dc)
    b, S, D = x.shape
    zc = z.shape[2]
    dx = np.zeros((b, S, D))
    dz = np.zeros((b, S, zc))
    _check(_load().csa_oracle_compress_bwd(b, S, D, ratio, span, zc, _ptr(x), _ptr(z), _ptr(dc),
                                           _ptr(dx), _ptr(dz)), "compress_bwd")
    return dx, dz


def index_scores(q_i_rows, k_i, w_rows, ratio, rows, doc=None):
    """Dense indexer scores of the listed rows.

    q_i_rows [n,HI,DI], w_rows [n,HI] hold the listed query rows; k_i is
    [b,n_c,DI]; rows [n,2] lists (batch, t); doc [b,S] optional document ids.
    Returns I [n, n_c] (-inf where block j is not valid for t)."""
    q, k, w = _f64(q_i_rows), _f64(k_i), _f64(w_rows)
    rows, rb, rt = _rows(rows, None, None)
    n, HI, DI = q.shape
    nc = k.shape[1]
    out = np.zeros((n, nc))
    d, S = _doc(doc)
    _check(_load().csa_oracle_index_scores(nc, ratio, HI, DI, _ptr(q), _ptr(k), _ptr(w), n,
                                           _ptr(rb), _ptr(rt), S, _ptr(d), _ptr(out)), "index_scores")
    return out


def topk(scores, ratio, k, rows, doc=None):
    """One full top-k per row; returns (idx int32 [n,K'], score fp64 [n,K'])."""
    s = _f64(scores)
    rows, rb, rt = _rows(rows, None, None)
    n, nc = s.shape
    kp = min(k, nc)
    idx = np.zeros((n, kp), dtype=np.int32)
    sc = np.zeros((n, kp))
    d, S = _doc(doc)
    _check(_load().csa_oracle_topk(nc, ratio, k, n, _ptr(rb), _ptr(rt), S, _ptr(d), _ptr(s), _ptr(idx),
                                   _ptr(sc)), "topk")
    return idx, sc


def index_topk(q_i, k_i, w, ratio, k, rows=None, doc=None):
    """Scores + top-k for rows of full tensors q_i [b,S,HI,DI], w [b,S,HI]."""
    q_i, w = np.asarray(q_i), np.asarray(w)
    b, S = q_i.shape[:2]
    rows, rb, rt = _rows(rows, b, S)
    scores = index_scores(q_i[rb, rt], k_i, w[rb, rt], ratio, rows, doc)
    idx, sc = topk(scores, ratio, k, rows, doc)
    return idx, sc, scores


def attn_fwd(q_rows, kv, c, idx_rows, sink, scale, window, ratio, rows, doc=None):
    """Forward for listed rows.  q_rows [n,H,D]; idx_rows [n,K'] int32 or None.

    Returns (O [n,H,D], LSE [n,H])."""
    q, kv, c = _f64(q_rows), _f64(kv), _f64(c)
    rows, rb, rt = _rows(rows, None, None)
    n, H, D = q.shape
    b, S, _ = kv.shape
    nc = c.shape[1]
    if idx_rows is not None:
        idx_rows = np.ascontiguousarray(np.asarray(idx_rows, dtype=np.int32))
        kp = idx_rows.shape[1]
    else:
        kp = 0
    snk = None if sink is None else _f64(sink)
    o = np.zeros((n, H, D))
    lse = np.zeros((n, H))
    d, _ = _doc(doc)
    _check(_load().csa_oracle_attn_fwd(S, H, D, window, ratio, nc, kp, _ptr(q), _ptr(kv), _ptr(c),
                                       _ptr(idx_rows), _ptr(snk), float(scale), n, _ptr(rb),
                                       _ptr(rt), _ptr(d), _ptr(o), _ptr(lse)), "attn_fwd")
    return o, lse


def attn_bwd(q_rows, kv, c, idx_rows, sink, scale, window, ratio, rows, do_rows, doc=None):
    """Backward for listed rows.  Returns (dQ [n,H,D], dKV [b,S,D], dC [b,n_c,D], dsink [H])."""
    q, kv, c, do = _f64(q_rows), _f64(kv), _f64(c), _f64(do_rows)
    rows, rb, rt = _rows(rows, None, None)
    n, H, D = q.shape
    b, S, _ = kv.shape
    nc = c.shape[1]
    if idx_rows is not None:
        idx_rows = np.ascontiguousarray(np.asarray(idx_rows, dtype=np.int32))
        kp = idx_rows.shape[1]
    else:
        kp = 0
    snk = None if sink is None else _f64(sink)
    dq = np.zeros((n, H, D))
    dkv = np.zeros((b, S, D))
    dc = np.zeros((b, nc, D))
    dsink = np.zeros((H,))
    d, _ = _doc(doc)
    _check(_load().csa_oracle_attn_bwd(S, H, D, window, ratio, nc, kp, _ptr(q), _ptr(kv), _ptr(c),
                                       _ptr(idx_rows), _ptr(snk), float(scale), n, _ptr(rb),
                                       _ptr(rt), _ptr(d), _ptr(do), _ptr(dq), _ptr(dkv), _ptr(dc),
                                       _ptr(dsink)), "attn_bwd")
    return dq, dkv, dc, dsink


def all_rows(b, sq):
    return _rows(None, b, sq)[0]
