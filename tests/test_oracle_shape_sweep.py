"""The fp64 oracle against the dense NumPy formulation over a sweep of small
shapes, degenerate ones included: sequences shorter than or equal to the
ratio (no or one compressed row), ratio 1, spans longer than the sequence,
windows of 1 and longer than the sequence, K' larger than the number of
compressed rows, one head, several batch rows.  The two formulations share no
code: the oracle walks each query's explicit candidate list, the dense
formulation builds one masked logit matrix over [window rows | compressed
rows | sink].  CPU only.
"""
import numpy as np
import pytest

import oracle
from oracle import brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

# (b, S, H, D, ratio, span, window, topk)
SHAPES = [
    (1, 1, 2, 4, 4, 4, 3, 2),       # one token, no compressed row
    (1, 3, 2, 4, 4, 8, 2, 2),       # shorter than the ratio
    (2, 4, 1, 6, 4, 4, 1, 1),       # exactly one block, window 1
    (1, 5, 3, 4, 4, 8, 9, 3),       # one block, window longer than the sequence
    (2, 9, 2, 5, 1, 1, 3, 4),       # ratio 1: every token a block
    (1, 17, 2, 4, 2, 6, 4, 20),     # K' capped at n_c
    (3, 23, 2, 3, 3, 7, 5, 2),      # ragged tail, span not a multiple of the ratio
    (1, 40, 4, 8, 8, 16, 6, 3),     # span twice the ratio
    (2, 33, 1, 4, 4, 12, 40, 8),    # window beyond the sequence
    (1, 31, 3, 2, 5, 5, 2, 1),      # K' = 1
]
IDS = [f"b{b}_S{S}_H{H}_D{D}_r{r}_L{L}_W{W}_K{K}" for b, S, H, D, r, L, W, K in SHAPES]


def _rng(shape_id):
    return np.random.default_rng(1000 + shape_id)


@pytest.mark.parametrize("case", range(len(SHAPES)), ids=IDS)
def test_compress_fwd_bwd_sweep(case):
    b, S, H, D, r, L, W, K = SHAPES[case]
    g = _rng(case)
    for zc in (D, 1):
        x, z = g.standard_normal((b, S, D)), g.standard_normal((b, S, zc))
        nc = S // r
        c = oracle.compress(x, z, r, L)
        cb, _ = brute.compress(x, z, r, L)
        assert c.shape == (b, nc, D)
        np.testing.assert_allclose(c, cb, rtol=1e-13, atol=1e-13)
        dc = g.standard_normal((b, nc, D))
        dx, dz = oracle.compress_bwd(x, z, dc, r, L)
        dxb, dzb = brute.compress_bwd(x, z, dc, r, L)
        np.testing.assert_allclose(dx, dxb, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dz, dzb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", range(len(SHAPES)), ids=IDS)
def test_index_topk_sweep(case):
    b, S, H, D, r, L, W, K = SHAPES[case]
    g = _rng(case)
    HI, DI, nc = 2, 4, S // r
    q, k, w = g.standard_normal((b, S, HI, DI)), g.standard_normal((b, nc, DI)), g.standard_normal((b, S, HI))
    idx, sc, scores = oracle.index_topk(q, k, w, r, K)
    kp = min(K, nc)
    assert idx.reshape(b, S, -1).shape == (b, S, kp)
    if nc == 0:
        return
    Ib = brute.index_scores(q, k, w, r)
    np.testing.assert_allclose(scores.reshape(b, S, -1), Ib, rtol=1e-13, atol=1e-13)
    bidx, bsc = brute.topk(Ib, r, K)
    np.testing.assert_array_equal(idx.reshape(bidx.shape), bidx)
    np.testing.assert_allclose(sc.reshape(bsc.shape), bsc, rtol=1e-13, atol=1e-13)


def _index_rows(g, b, S, r, nc, kp):
    idx = np.full((b, S, kp), -1, dtype=np.int32)
    for bi in range(b):
        for t in range(S):
            nv = min((t + 1) // r, nc)
            m = min(kp, nv)
            if m:
                idx[bi, t, :m] = np.sort(g.choice(nv, m, replace=False))
    return idx


@pytest.mark.parametrize("case", range(len(SHAPES)), ids=IDS)
@pytest.mark.parametrize("mode", ["selected", "dense"])
def test_attention_fwd_bwd_sweep(case, mode):
    b, S, H, D, r, L, W, K = SHAPES[case]
    g = _rng(case)
    nc = S // r
    kp = min(K, nc)
    q, kv, c = g.standard_normal((b, S, H, D)), g.standard_normal((b, S, D)), g.standard_normal((b, nc, D))
    sink, do = g.standard_normal(H), g.standard_normal((b, S, H, D))
    idx = _index_rows(g, b, S, r, nc, kp) if (mode == "selected" and kp > 0) else None
    scale = 0.37
    rows = oracle.all_rows(b, S)
    flat = None if idx is None else idx.reshape(b * S, -1)
    o, lse = oracle.attn_fwd(q.reshape(b * S, H, D), kv, c, flat, sink, scale, W, r, rows)
    ob, lseb, _, _ = brute.attn_fwd(q, kv, c, idx, sink, scale, W, r)
    np.testing.assert_allclose(o.reshape(q.shape), ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse.reshape(b, S, H), lseb, rtol=1e-12, atol=1e-12)
    got = oracle.attn_bwd(q.reshape(b * S, H, D), kv, c, flat, sink, scale, W, r, rows, do.reshape(b * S, H, D))
    ref = brute.attn_bwd(q, kv, c, idx, sink, scale, W, r, do)
    np.testing.assert_allclose(got[0].reshape(q.shape), ref[0], rtol=1e-11, atol=1e-12)
    for gg, rf in zip(got[1:], ref[1:]):
        np.testing.assert_allclose(gg, rf, rtol=1e-11, atol=1e-12)
