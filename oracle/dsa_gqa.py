"""fp64 oracle of the simplified DSA over grouped-query attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Megatron-LM PR #7152 (its description and commit messages): a learned
indexer with a single head and no per-head weights scores every earlier
key at full resolution, I[t, j] = ReLU(<q_i[t], k_i[j]>) for j <= t, and one
full top-k per query selects K' keys; attention then runs over the selected
keys only, with grouped-query attention: query head h reads key/value head
g = h // (H / H_kv), keys and values being separate tensors.  The indexer is
the compressed indexer of ``oracle.index_topk`` with ratio 1, one head and
unit weights (a block is a token).

Readings: a selected slot is valid when 0 <= j <= t (the causal rule of
ratio 1); a repeated index counts once per slot; no window rows and no sink;
a query with no valid slot gets a zero output, LSE = -inf and no gradient.

Plain NumPy, one query row at a time.
"""
from __future__ import annotations

import numpy as np


def _support(idx_row, t):
    idx_row = np.asarray(idx_row, dtype=np.int64)
    return idx_row[(idx_row >= 0) & (idx_row <= t)]


def _rows(rows, b, S):
    if rows is None:
        return [(bi, t) for bi in range(b) for t in range(S)]
    return [(int(bi), int(t)) for bi, t in rows]


def fwd(q, k, v, idx, scale, rows=None):
    """q [b,S,H,dk], k [b,S,Hkv,dk], v [b,S,Hkv,dv], idx [b,S,K'].

    Returns (out [b,S,H,dv], lse [b,S,H]) for the listed (batch, t) rows
    (all rows by default; the others stay 0 / -inf)."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    b, S, H, dk = q.shape
    hkv, dv = k.shape[2], v.shape[3]
    grp = H // hkv
    out = np.zeros((b, S, H, dv))
    lse = np.full((b, S, H), -np.inf)
    for bi, t in _rows(rows, b, S):
        js = _support(idx[bi, t], t)
        if len(js) == 0:
            continue
        for h in range(H):
            g = h // grp
            s = scale * (k[bi, js, g] @ q[bi, t, h])
            m = s.max()
            e = np.exp(s - m)
            lse[bi, t, h] = m + np.log(e.sum())
            out[bi, t, h] = (e / e.sum()) @ v[bi, js, g]
    return out, lse


def bwd(q, k, v, idx, scale, out, lse, dout, rows=None):
    """Gradients (dq, dk, dv) of sum(dout * out) over the listed rows (all by
    default; rows not listed contribute nothing)."""
    q, k, v, out, lse, dout = (np.asarray(a, np.float64) for a in (q, k, v, out, lse, dout))
    b, S, H, dk = q.shape
    hkv = k.shape[2]
    grp = H // hkv
    dq, dkk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for bi, t in _rows(rows, b, S):
        js = _support(idx[bi, t], t)
        if len(js) == 0:
            continue
        for h in range(H):
            g = h // grp
            s = scale * (k[bi, js, g] @ q[bi, t, h])
            p = np.exp(s - lse[bi, t, h])
            dp = v[bi, js, g] @ dout[bi, t, h]
            delta = dout[bi, t, h] @ out[bi, t, h]
            ds = p * (dp - delta)
            dq[bi, t, h] = scale * ds @ k[bi, js, g]
            np.add.at(dkk[bi, :, g], js, scale * ds[:, None] * q[bi, t, h][None, :])
            np.add.at(dvv[bi, :, g], js, p[:, None] * dout[bi, t, h][None, :])
    return dq, dkk, dvv
