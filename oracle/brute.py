"""Dense NumPy fp64 formulation of the CSA hot path (tiny inputs only).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  This second
formulation is written independently of ``csa_oracle.c``: instead of explicit
candidate lists it builds dense masked matrices.

* Compressor: a pooling-membership mask ``[n_c, S]`` and a masked softmax over
  the sequence axis per channel (Megatron-LM PR #6400, review thread on the
  compressor's fp32 pooling weights).
* Indexer: the dense ``[S, n_c]`` score matrix with the compressed causal mask
  ``j >= (t+1)//ratio -> -inf`` (same PR, thread on the per-forward causal
  mask), then a lexicographic sort.
* Attention: one logit matrix per head over the unified key axis of length
  ``S + n_c`` (raw KV rows first, compressed rows after them, as in the same
  PR's index space with the compressed offset ``S``) plus one sink column
  (torchtitan PR #4452: window, selected compressed rows and sink share one
  softmax).  Multiplicity matrices count how many slots select each key, so a
  repeated index in one row counts once per slot.
* Backward: the matrix form of the softmax-with-sink gradient.
* Packed documents (``doc`` [b, S]): equality masks ``doc[t] == doc[u]`` on the
  window and ``doc[t] == doc[j*ratio]`` on the indexer's blocks (torchtitan
  PR #4452, its description of packed documents); dense mode (no index rows)
  uses the indexer's block rule, given index rows are taken as they are.
"""
from __future__ import annotations

import numpy as np


def pool_membership(S: int, ratio: int, span: int) -> np.ndarray:
    """M[j, u] = 1 iff token u lies in the pooling span of block j."""
    nc = S // ratio
    j = np.arange(nc)[:, None]
    u = np.arange(S)[None, :]
    return ((u < (j + 1) * ratio) & (u >= (j + 1) * ratio - span)).astype(np.float64)


def compress(x, z, ratio, span):
    x = np.asarray(x, np.float64)
    z = np.asarray(z, np.float64)
    b, S, D = x.shape
    zb = np.broadcast_to(z, (b, S, D))
    M = pool_membership(S, ratio, span)                      # [nc, S]
    logits = np.where(M[None, :, :, None] > 0, zb[:, None, :, :], -np.inf)  # [b,nc,S,D]
    mx = logits.max(axis=2, keepdims=True)
    e = np.exp(logits - mx)
    alpha = e / e.sum(axis=2, keepdims=True)
    return np.einsum("bjuc,buc->bjc", alpha, x), alpha


def compress_bwd(x, z, dc, ratio, span):
    x = np.asarray(x, np.float64)
    z = np.asarray(z, np.float64)
    dc = np.asarray(dc, np.float64)
    c, alpha = compress(x, z, ratio, span)
    dx = np.einsum("bjuc,bjc->buc", alpha, dc)
    # d alpha_u / d z_v = alpha_u (delta_uv - alpha_v), so
    # dZ[u,c] = sum_j alpha[j,u,c] dC[j,c] (x[u,c] - C[j,c])
    dz_full = alpha * (dc[:, :, None, :] * x[:, None, :, :] - (dc * c)[:, :, None, :])
    dz = dz_full.sum(axis=1)
    if z.shape[2] == 1:
        dz = dz.sum(axis=2, keepdims=True)
    return dx, dz


def compressed_valid(S: int, ratio: int) -> np.ndarray:
    """V[t, j] = block j is causally valid for query t."""
    nc = S // ratio
    t = np.arange(S)[:, None]
    j = np.arange(nc)[None, :]
    return j < (t + 1) // ratio


def block_valid(b, S, ratio, doc=None):
    """V[b, t, j]: block j is valid for query t (causal, and with doc in t's document)."""
    V = np.broadcast_to(compressed_valid(S, ratio)[None], (b, S, S // ratio))
    if doc is None:
        return V
    doc = np.asarray(doc)
    nc = S // ratio
    return V & (doc[:, :, None] == doc[:, None, np.arange(nc) * ratio])


def index_scores(q_i, k_i, w, ratio, doc=None):
    q_i = np.asarray(q_i, np.float64)   # [b,S,HI,DI]
    k_i = np.asarray(k_i, np.float64)   # [b,nc,DI]
    w = np.asarray(w, np.float64)       # [b,S,HI]
    b, S = q_i.shape[:2]
    dots = np.einsum("bthe,bje->bthj", q_i, k_i)
    I = np.einsum("bth,bthj->btj", w, np.maximum(dots, 0.0))
    return np.where(block_valid(b, S, ratio, doc), I, -np.inf)


def topk(I, ratio, k, doc=None):
    b, S, nc = I.shape
    kp = min(k, nc)
    V = block_valid(b, S, ratio, doc)
    idx = np.full((b, S, kp), -1, dtype=np.int32)
    sc = np.full((b, S, kp), -np.inf)
    for bi in range(b):
        for t in range(S):
            js = np.nonzero(V[bi, t])[0]
            order = np.lexsort((js, -I[bi, t, js]))     # primary: score desc, then index asc
            sel = np.sort(js[order[:kp]])
            idx[bi, t, :len(sel)] = sel
            sc[bi, t, :len(sel)] = I[bi, t, sel]
    return idx, sc


def key_multiplicity(S, nc, window, ratio, idx, doc=None):
    """N[b, t, key] over the unified axis [S + nc]: how many candidates of
    query t point at each key (window rows once, compressed rows once per
    valid slot; idx None = every valid compressed row once)."""
    t = np.arange(S)[:, None]
    u = np.arange(S)[None, :]
    win = ((u <= t) & (u > t - window)).astype(np.float64)[None]    # [1, S, S]
    if doc is not None:
        d = np.asarray(doc)
        win = win * (d[:, :, None] == d[:, None, :])                 # [b, S, S]
    V = compressed_valid(S, ratio)
    if idx is None:
        bd = 1 if doc is None else np.asarray(doc).shape[0]
        comp = block_valid(bd, S, ratio, doc).astype(np.float64)     # [bd, S, nc]
        b = bd
    else:
        idx = np.asarray(idx)
        b = idx.shape[0]
        comp = np.zeros((b, S, nc))
        for bi in range(b):
            for tt in range(S):
                for j in idx[bi, tt]:
                    if 0 <= j < nc and V[tt, j]:
                        comp[bi, tt, j] += 1.0
    bb = max(comp.shape[0], win.shape[0])
    return np.concatenate([np.broadcast_to(win, (bb, S, S)), np.broadcast_to(comp, (bb, S, nc))], axis=2), b


def attn_fwd(q, kv, c, idx, sink, scale, window, ratio, doc=None):
    """Returns (O [b,S,H,D], LSE [b,S,H], P [b,S,H,S+nc], Psink [b,S,H])."""
    q = np.asarray(q, np.float64)
    kv = np.asarray(kv, np.float64)
    c = np.asarray(c, np.float64)
    b, S, H, D = q.shape
    nc = c.shape[1]
    N, _ = key_multiplicity(S, nc, window, ratio, idx, doc)
    N = np.broadcast_to(N, (b, S, S + nc))
    keys = np.concatenate([kv, c], axis=1)                           # [b, S+nc, D]
    logits = scale * np.einsum("bthd,bkd->bthk", q, keys)
    sink_col = (np.full((H,), -np.inf) if sink is None else np.asarray(sink, np.float64))
    # weight each key by its multiplicity: exp(l) * N
    with np.errstate(divide="ignore"):
        logN = np.log(N)[:, :, None, :]
    full = logits + logN
    mx = np.maximum(full.max(axis=3), sink_col[None, None, :])
    den = np.exp(full - mx[..., None]).sum(axis=3) + np.exp(sink_col[None, None, :] - mx)
    lse = mx + np.log(den)
    P = np.exp(full - lse[..., None])                               # includes multiplicity
    o = np.einsum("bthk,bkd->bthd", P, keys)
    psink = np.exp(sink_col[None, None, :] - lse)
    return o, lse, P, psink


def attn_bwd(q, kv, c, idx, sink, scale, window, ratio, do, doc=None):
    """Returns (dQ, dKV, dC, dsink)."""
    q = np.asarray(q, np.float64)
    kv = np.asarray(kv, np.float64)
    c = np.asarray(c, np.float64)
    do = np.asarray(do, np.float64)
    S = q.shape[1]
    o, lse, P, psink = attn_fwd(q, kv, c, idx, sink, scale, window, ratio, doc)
    keys = np.concatenate([kv, c], axis=1)
    delta = np.einsum("bthd,bthd->bth", do, o)
    dP = np.einsum("bthd,bkd->bthk", do, keys)
    dl = P * (dP - delta[..., None])
    dq = scale * np.einsum("bthk,bkd->bthd", dl, keys)
    dkeys = np.einsum("bthk,bthd->bkd", P, do) + scale * np.einsum("bthk,bthd->bkd", dl, q)
    dsink = -(psink * delta).sum(axis=(0, 1)) if sink is not None else None
    return dq, dkeys[:, :S], dkeys[:, S:], dsink
