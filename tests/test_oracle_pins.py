"""Pins of the fp64 oracle against facts fixed outside it.

Each test ties one oracle function to something other than itself: a closed
form, a textbook or library routine (numpy sorting, torch's scaled dot-product
attention, torch autograd), central finite differences, or the independent
dense NumPy formulation in ``oracle/brute.py``.  Chosen so that a dropped term,
a wrong sign or index, or a transposed operand in the oracle fails one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute

RNG = np.random.default_rng(1234)


def rnd(*shape, s=1.0):
    return RNG.standard_normal(shape) * s


# ----------------------------------------------------------------- compressor
@pytest.mark.parametrize("ratio,span,zc", [(4, 4, 8), (4, 8, 8), (4, 8, 1), (3, 7, 8), (8, 8, 1)])
def test_compress_matches_dense_formulation(ratio, span, zc):
    x, z = rnd(2, 37, 8), rnd(2, 37, zc)
    c = oracle.compress(x, z, ratio, span)
    cb, _ = brute.compress(x, z, ratio, span)
    assert c.shape == (2, 37 // ratio, 8)
    np.testing.assert_allclose(c, cb, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("ratio,span", [(4, 4), (4, 8), (5, 12)])
def test_compress_weights_sum_to_one(ratio, span):
    # X == 1 everywhere: the pooled row is sum_u alpha_u = 1 for every block
    z = rnd(1, 40, 6, s=3.0)
    c = oracle.compress(np.ones((1, 40, 6)), z, ratio, span)
    np.testing.assert_allclose(c, 1.0, rtol=0, atol=1e-14)


def test_compress_constant_scores_is_mean_pooling():
    # constant scores give uniform weights: the textbook mean of each span,
    # clipped at the sequence start for the first block of an overlapping span
    x = rnd(1, 32, 5)
    c = oracle.compress(x, np.full((1, 32, 5), 0.7), 4, 8)
    for j in range(8):
        lo, hi = max(0, (j + 1) * 4 - 8), (j + 1) * 4
        np.testing.assert_allclose(c[0, j], x[0, lo:hi].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_compress_ratio_one_is_identity():
    x, z = rnd(1, 9, 4), rnd(1, 9, 4)
    np.testing.assert_allclose(oracle.compress(x, z, 1, 1), x, rtol=0, atol=0)


def test_compress_row_score_broadcasts():
    x, z1 = rnd(1, 24, 6), rnd(1, 24, 1)
    np.testing.assert_allclose(oracle.compress(x, z1, 4, 8),
                               oracle.compress(x, np.repeat(z1, 6, axis=2), 4, 8), rtol=1e-14)


def test_compress_two_rows_closed_form():
    # one block of two rows: alpha_0 = sigmoid(z0 - z1)
    x, z = rnd(1, 2, 3), rnd(1, 2, 3)
    a0 = 1.0 / (1.0 + np.exp(-(z[0, 0] - z[0, 1])))
    np.testing.assert_allclose(oracle.compress(x, z, 2, 2)[0, 0], a0 * x[0, 0] + (1 - a0) * x[0, 1],
                               rtol=1e-14)


@pytest.mark.parametrize("ratio,span,zc", [(4, 4, 8), (4, 8, 8), (4, 8, 1)])
def test_compress_bwd_finite_differences(ratio, span, zc):
    S, D = 32, 8
    x, z, dc = rnd(1, S, D), rnd(1, S, zc), rnd(1, S // ratio, D)
    dx, dz = oracle.compress_bwd(x, z, dc, ratio, span)
    h = 1e-6

    def loss(xx, zz):
        return float((oracle.compress(xx, zz, ratio, span) * dc).sum())

    num_dx = np.zeros_like(x)
    for u in range(S):
        for c in range(D):
            e = np.zeros_like(x); e[0, u, c] = h
            num_dx[0, u, c] = (loss(x + e, z) - loss(x - e, z)) / (2 * h)
    num_dz = np.zeros_like(z)
    for u in range(S):
        for c in range(zc):
            e = np.zeros_like(z); e[0, u, c] = h
            num_dz[0, u, c] = (loss(x, z + e) - loss(x, z - e)) / (2 * h)
    assert np.abs(dx - num_dx).max() <= 1e-6 * np.abs(num_dx).max()
    assert np.abs(dz - num_dz).max() <= 1e-6 * np.abs(num_dz).max()
    bdx, bdz = brute.compress_bwd(x, z, dc, ratio, span)
    np.testing.assert_allclose(dx, bdx, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dz, bdz, rtol=1e-12, atol=1e-13)


def test_compress_tail_rows_get_no_gradient():
    # S not a multiple of ratio: the trailing rows belong to no block
    x, z, dc = rnd(1, 23, 4), rnd(1, 23, 4), rnd(1, 5, 4)
    dx, dz = oracle.compress_bwd(x, z, dc, 4, 4)
    assert np.all(dx[0, 20:] == 0) and np.all(dz[0, 20:] == 0)
    assert np.all(dx[0, :20] != 0)


# ------------------------------------------------------------ indexer / top-k
def _index_inputs(b, S, nc, HI, DI):
    return rnd(b, S, HI, DI), rnd(b, nc, DI), rnd(b, S, HI)


@pytest.mark.parametrize("k", [1, 5, 16, 40])
def test_index_topk_matches_dense_formulation(k):
    b, S, r, HI, DI = 2, 64, 4, 3, 8
    q, kk, w = _index_inputs(b, S, S // r, HI, DI)
    idx, sc, scores = oracle.index_topk(q, kk, w, r, k)
    Ib = brute.index_scores(q, kk, w, r)
    np.testing.assert_allclose(scores.reshape(b, S, -1), Ib, rtol=1e-13, atol=1e-13)
    bidx, bsc = brute.topk(Ib, r, k)
    np.testing.assert_array_equal(idx.reshape(bidx.shape), bidx)
    np.testing.assert_allclose(sc.reshape(bsc.shape), bsc, rtol=1e-13, atol=1e-13)


def test_index_scores_textbook_single_head():
    # one head with unit weight and positive dot products: the score is q.k
    S, r, DI = 40, 4, 6
    q = np.abs(rnd(1, S, 1, DI)) + 0.1
    kk = np.abs(rnd(1, S // r, DI)) + 0.1
    w = np.ones((1, S, 1))
    _, _, scores = oracle.index_topk(q, kk, w, r, 4)
    ref = q[0, :, 0, :] @ kk[0].T
    valid = np.arange(S // r)[None, :] < (np.arange(S)[:, None] + 1) // r
    np.testing.assert_allclose(scores[valid], ref[valid], rtol=1e-14)
    assert np.all(np.isneginf(scores[~valid]))


def test_topk_matches_library_sort():
    # ranking by numpy's stable argsort of -score (ties -> lower index first)
    S, r, k = 80, 4, 7
    q, kk, w = _index_inputs(1, S, S // r, 2, 5)
    idx, _, scores = oracle.index_topk(q, kk, w, r, k)
    for t in range(S):
        nv = (t + 1) // r
        order = np.argsort(-scores[t, :nv], kind="stable")[:min(k, nv)]
        ref = np.sort(order)
        got = idx[t][idx[t] >= 0]
        np.testing.assert_array_equal(got, ref)
        assert np.all(idx[t][len(got):] == -1)


def test_topk_k1_is_argmax_lowest_index():
    S, r = 48, 4
    q, kk, w = _index_inputs(1, S, S // r, 2, 4)
    kk[0, 3] = kk[0, 7]                     # two identical keys -> exact tie
    idx, _, scores = oracle.index_topk(q, kk, w, r, 1)
    for t in range(S):
        nv = (t + 1) // r
        if nv == 0:
            assert idx[t, 0] == -1
        else:
            assert idx[t, 0] == int(np.argmax(scores[t, :nv]))   # numpy: first maximum


def test_topk_all_valid_when_k_covers_prefix():
    # K' >= n_valid(t): every valid block, in order, then K' - n_valid slots of -1
    S, r, k = 64, 4, 16
    q, kk, w = _index_inputs(1, S, S // r, 2, 4)
    idx, _, _ = oracle.index_topk(q, kk, w, r, k)
    for t in range(S):
        nv = (t + 1) // r
        np.testing.assert_array_equal(idx[t, :nv], np.arange(nv))
        assert np.all(idx[t, nv:] == -1) and idx.shape[1] == 16


def test_topk_zero_keys_ties_to_lowest_index():
    # k_i == 0: every score is 0 (or -0 with negative weights) -> all ties
    S, r, k = 64, 4, 5
    q, _, w = _index_inputs(1, S, S // r, 3, 4)
    idx, sc, _ = oracle.index_topk(q, np.zeros((1, S // r, 4)), -np.abs(w), r, k)
    for t in range(S):
        m = min(k, (t + 1) // r)
        np.testing.assert_array_equal(idx[t, :m], np.arange(m))
        assert np.all(idx[t, m:] == -1)
        assert np.all(sc[t, :m] == 0.0)


def test_topk_kprime_caps_at_n_compressed():
    S, r = 32, 4
    q, kk, w = _index_inputs(1, S, S // r, 2, 4)
    idx, _, _ = oracle.index_topk(q, kk, w, r, 100)
    assert idx.shape[1] == S // r


def test_index_rows_subset_matches_full():
    b, S, r = 2, 48, 4
    q, kk, w = _index_inputs(b, S, S // r, 2, 4)
    idx_full, sc_full, _ = oracle.index_topk(q, kk, w, r, 6)
    rows = np.array([[1, 47], [0, 3], [1, 10], [0, 0]])
    idx_s, sc_s, _ = oracle.index_topk(q, kk, w, r, 6, rows=rows)
    flat = rows[:, 0] * S + rows[:, 1]
    np.testing.assert_array_equal(idx_s, idx_full[flat])
    np.testing.assert_array_equal(sc_s, sc_full[flat])


# --------------------------------------------------------------- attention fwd
def _attn_case(b=2, S=32, H=3, D=6, r=4, W=5, kp=4, seed_idx=True, dup=False, junk=False):
    nc = S // r
    q, kv, c = rnd(b, S, H, D), rnd(b, S, D), rnd(b, nc, D)
    sink = rnd(H)
    idx = None
    if seed_idx:
        idx = np.full((b, S, kp), -1, dtype=np.int32)
        for bi in range(b):
            for t in range(S):
                nv = (t + 1) // r
                m = min(kp, nv)
                if m:
                    idx[bi, t, :m] = np.sort(RNG.choice(nv, m, replace=False))
                if dup and m >= 2:
                    idx[bi, t, 1] = idx[bi, t, 0]
                if junk:
                    idx[bi, t, -1] = nc + 3 if t % 2 else (t + 1) // r
    return q, kv, c, idx, sink


def _fwd(q, kv, c, idx, sink, scale, W, r):
    b, S = q.shape[:2]
    rows = oracle.all_rows(b, S)
    o, lse = oracle.attn_fwd(q.reshape(b * S, *q.shape[2:]), kv, c,
                             None if idx is None else idx.reshape(b * S, -1), sink, scale, W, r, rows)
    return o.reshape(q.shape), lse.reshape(b, S, -1)


@pytest.mark.parametrize("kw", [dict(), dict(dup=True), dict(junk=True), dict(seed_idx=False),
                                dict(W=1), dict(W=64)])
@pytest.mark.parametrize("with_sink", [True, False])
def test_attn_fwd_matches_dense_formulation(kw, with_sink):
    q, kv, c, idx, sink = _attn_case(**kw)
    W = kw.get("W", 5)
    sink = sink if with_sink else None
    o, lse = _fwd(q, kv, c, idx, sink, 0.4, W, 4)
    ob, lseb, _, _ = brute.attn_fwd(q, kv, c, idx, sink, 0.4, W, 4)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-12)


def test_attn_fwd_against_torch_sdpa():
    # the sink becomes one extra key with a zero value row and an extra feature
    # that carries sink_h / scale; torch's SDPA (fp64, CPU, explicit mask) then
    # computes exactly the sink-augmented softmax attention.
    b, S, H, D, r, W = 1, 24, 2, 5, 4, 6
    q, kv, c, idx, sink = _attn_case(b=b, S=S, H=H, D=D, r=r, W=W, kp=3)
    scale = 0.37
    nc = S // r
    o, lse = _fwd(q, kv, c, idx, sink, scale, W, r)
    keys = np.concatenate([kv[0], c[0]], axis=0)                       # [S+nc, D]
    mask = np.zeros((S, S + nc + 1), dtype=bool)
    for t in range(S):
        mask[t, max(0, t - W + 1):t + 1] = True
        for j in idx[0, t]:
            if 0 <= j < (t + 1) // r:
                mask[t, S + j] = True
        mask[t, -1] = True
    qa = np.concatenate([q[0], np.ones((S, H, 1))], axis=2)             # [S,H,D+1]
    out = np.zeros((S, H, D))
    for h in range(H):
        ka = np.concatenate([np.concatenate([keys, np.zeros((S + nc, 1))], 1),
                             np.concatenate([np.zeros((1, D)), [[sink[h] / scale]]], 1)], 0)
        va = np.concatenate([keys, np.zeros((1, D))], 0)
        qq = torch.tensor(qa[:, h], dtype=torch.float64)[None, None]
        res = torch.nn.functional.scaled_dot_product_attention(
            qq, torch.tensor(ka)[None, None], torch.tensor(np.concatenate([va, np.zeros((S + nc + 1, 1))], 1))[None, None],
            attn_mask=torch.tensor(mask)[None, None], scale=scale)
        out[:, h] = res[0, 0, :, :D].numpy()
    np.testing.assert_allclose(o[0], out, rtol=1e-12, atol=1e-12)


def test_attn_mass_plus_sink_is_one():
    q, kv, c, idx, sink = _attn_case()
    scale, W, r = 0.5, 5, 4
    o, lse = _fwd(q, kv, c, idx, sink, scale, W, r)
    b, S, H, D = q.shape
    for bi in range(b):
        for t in range(S):
            rows = [kv[bi, u] for u in range(max(0, t - W + 1), t + 1)]
            rows += [c[bi, j] for j in idx[bi, t] if 0 <= j < (t + 1) // r]
            R = np.array(rows)
            for h in range(H):
                mass = np.exp(scale * R @ q[bi, t, h] - lse[bi, t, h]).sum()
                assert abs(mass + np.exp(sink[h] - lse[bi, t, h]) - 1.0) < 1e-12


def test_attn_first_query_closed_form():
    # t = 0 sees only its own raw row (no block is valid yet):
    # O = sigmoid(s - sink) kv_0 and LSE = logaddexp(sink, s), s = scale <q, kv_0>
    q, kv, c, idx, sink = _attn_case()
    scale = 0.3
    o, lse = _fwd(q, kv, c, idx, sink, scale, 5, 4)
    for bi in range(2):
        s = scale * q[bi, 0] @ kv[bi, 0]
        np.testing.assert_allclose(lse[bi, 0], np.logaddexp(sink, s), rtol=1e-14)
        np.testing.assert_allclose(o[bi, 0], (1 / (1 + np.exp(-(s - sink))))[:, None] * kv[bi, 0],
                                   rtol=1e-13, atol=1e-14)


def test_attn_window_one_no_blocks_closed_form_every_query():
    q, kv, c, idx, sink = _attn_case()
    scale = 0.3
    o, lse = _fwd(q, kv, c, np.full_like(idx, -1), sink, scale, 1, 4)
    s = scale * np.einsum("bthd,btd->bth", q, kv)
    # an LSE near 0 is the difference of terms of size ~1: allow their rounding
    np.testing.assert_allclose(lse, np.logaddexp(sink[None, None], s), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o, (1 / (1 + np.exp(-(s - sink))))[..., None] * kv[:, :, None],
                               rtol=1e-13, atol=1e-14)


def test_attn_full_topk_equals_dense_compressed_mode():
    # K' >= n_valid(t): selecting every valid block equals the dense mode
    q, kv, c, _, sink = _attn_case()
    S, r = 32, 4
    nc = S // r
    idx = np.full((2, S, nc), -1, dtype=np.int32)
    for t in range(S):
        nv = (t + 1) // r
        idx[:, t, :nv] = np.arange(nv)
    o1, l1 = _fwd(q, kv, c, idx, sink, 0.4, 5, r)
    o2, l2 = _fwd(q, kv, c, None, sink, 0.4, 5, r)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_attn_slot_permutation_invariance():
    q, kv, c, idx, sink = _attn_case()
    perm = RNG.permutation(idx.shape[2])
    o1, l1 = _fwd(q, kv, c, idx, sink, 0.4, 5, 4)
    o2, l2 = _fwd(q, kv, c, idx[:, :, perm], sink, 0.4, 5, 4)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_attn_no_sink_is_plain_softmax_attention():
    q, kv, c, idx, _ = _attn_case(b=1, S=16, H=2, D=4)
    o, lse = _fwd(q, kv, c, idx, None, 0.5, 5, 4)
    t, h = 13, 1
    rows = [kv[0, u] for u in range(9, 14)] + [c[0, j] for j in idx[0, t] if 0 <= j < 3]
    R = np.array(rows)
    p = torch.softmax(torch.tensor(0.5 * R @ q[0, t, h]), dim=0).numpy()
    np.testing.assert_allclose(o[0, t, h], p @ R, rtol=1e-13)


# --------------------------------------------------------------- attention bwd
def _bwd(q, kv, c, idx, sink, scale, W, r, do):
    b, S = q.shape[:2]
    rows = oracle.all_rows(b, S)
    dq, dkv, dc, dsink = oracle.attn_bwd(q.reshape(b * S, *q.shape[2:]), kv, c,
                                         None if idx is None else idx.reshape(b * S, -1), sink,
                                         scale, W, r, rows, do.reshape(b * S, *do.shape[2:]))
    return dq.reshape(q.shape), dkv, dc, dsink


@pytest.mark.parametrize("kw", [dict(), dict(dup=True, junk=True), dict(seed_idx=False)])
def test_attn_bwd_matches_dense_formulation(kw):
    q, kv, c, idx, sink = _attn_case(**kw)
    do = rnd(*q.shape)
    got = _bwd(q, kv, c, idx, sink, 0.4, 5, 4, do)
    ref = brute.attn_bwd(q, kv, c, idx, sink, 0.4, 5, 4, do)
    for g, rf in zip(got, ref):
        np.testing.assert_allclose(g, rf, rtol=1e-11, atol=1e-12)


def test_attn_bwd_finite_differences():
    b, S, H, D, r, W, kp = 1, 24, 2, 5, 4, 4, 2
    q, kv, c, idx, sink = _attn_case(b=b, S=S, H=H, D=D, r=r, W=W, kp=kp, dup=True)
    do = rnd(*q.shape)
    scale = 0.45
    dq, dkv, dc, dsink = _bwd(q, kv, c, idx, sink, scale, W, r, do)

    def loss(q_, kv_, c_, s_):
        o, _ = _fwd(q_, kv_, c_, idx, s_, scale, W, r)
        return float((o * do).sum())

    h = 1e-6

    def num(arr, which):
        g = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            e = np.zeros_like(arr); e[i] = h
            args_p = [q, kv, c, sink]; args_m = [q, kv, c, sink]
            args_p[which] = arr + e; args_m[which] = arr - e
            g[i] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        return g

    for got, arr, which in ((dq, q, 0), (dkv, kv, 1), (dc, c, 2), (dsink, sink, 3)):
        ref = num(arr, which)
        assert np.abs(got - ref).max() <= 1e-6 * np.abs(ref).max(), which


def test_attn_bwd_against_torch_autograd():
    # a gather-based torch fp64 re-formulation differentiated by autograd
    b, S, H, D, r, W, kp = 2, 20, 3, 4, 4, 3, 3
    q, kv, c, idx, sink = _attn_case(b=b, S=S, H=H, D=D, r=r, W=W, kp=kp, dup=True, junk=True)
    do = rnd(*q.shape)
    scale = 0.6
    got = _bwd(q, kv, c, idx, sink, scale, W, r, do)
    tq, tkv, tc, ts = (torch.tensor(a, requires_grad=True) for a in (q, kv, c, sink))
    out = torch.zeros(b, S, H, D, dtype=torch.float64)
    outs = []
    for bi in range(b):
        for t in range(S):
            rows = [tkv[bi, u] for u in range(max(0, t - W + 1), t + 1)]
            rows += [tc[bi, int(j)] for j in idx[bi, t] if 0 <= j < (t + 1) // r]
            R = torch.stack(rows)
            logits = scale * tq[bi, t] @ R.T                      # [H, n]
            full = torch.cat([logits, ts[:, None]], dim=1)
            p = torch.softmax(full, dim=1)[:, :-1]
            outs.append(p @ R)
    out = torch.stack(outs).reshape(b, S, H, D)
    (out * torch.tensor(do)).sum().backward()
    for g, t_ in zip(got, (tq, tkv, tc, ts)):
        np.testing.assert_allclose(g, t_.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_attn_bwd_sink_closed_form():
    # dsink_h = -sum_{b,t} exp(sink_h - LSE) <dO, O>, with O, LSE from the forward
    q, kv, c, idx, sink = _attn_case()
    do = rnd(*q.shape)
    o, lse = _fwd(q, kv, c, idx, sink, 0.4, 5, 4)
    _, _, _, dsink = _bwd(q, kv, c, idx, sink, 0.4, 5, 4, do)
    ref = -(np.exp(sink[None, None] - lse) * np.einsum("bthd,bthd->bth", do, o)).sum(axis=(0, 1))
    np.testing.assert_allclose(dsink, ref, rtol=1e-12)


def test_attn_bwd_linear_in_dout():
    q, kv, c, idx, sink = _attn_case()
    d1, d2 = rnd(*q.shape), rnd(*q.shape)
    g1 = _bwd(q, kv, c, idx, sink, 0.4, 5, 4, d1)
    g2 = _bwd(q, kv, c, idx, sink, 0.4, 5, 4, d2)
    g3 = _bwd(q, kv, c, idx, sink, 0.4, 5, 4, 2.5 * d1 + d2)
    for a, bb, cc in zip(g1, g2, g3):
        np.testing.assert_allclose(cc, 2.5 * a + bb, rtol=1e-10, atol=1e-12)


def test_attn_bwd_shared_block_accumulates():
    # every query that can selects block 0: dC[0] collects all of them
    b, S, r, W = 1, 16, 4, 2
    q, kv, c, _, sink = _attn_case(b=b, S=S, W=W)
    idx = np.full((b, S, 2), -1, dtype=np.int32)
    idx[0, 3:, 0] = 0
    do = rnd(*q.shape)
    dq, dkv, dc, dsink = _bwd(q, kv, c, idx, sink, 0.4, W, r, do)
    assert np.all(dc[0, 1:] == 0) and np.abs(dc[0, 0]).sum() > 0
    ref = brute.attn_bwd(q, kv, c, idx, sink, 0.4, W, r, do)
    np.testing.assert_allclose(dc, ref[2], rtol=1e-12, atol=1e-13)
    # contributions from one query at a time add up to the joint result
    acc = np.zeros_like(dc)
    for t in range(S):
        m = np.zeros_like(do); m[0, t] = do[0, t]
        acc += _bwd(q, kv, c, idx, sink, 0.4, W, r, m)[2]
    np.testing.assert_allclose(acc, dc, rtol=1e-12, atol=1e-13)


def test_attn_rows_subset_matches_full():
    q, kv, c, idx, sink = _attn_case()
    o, lse = _fwd(q, kv, c, idx, sink, 0.4, 5, 4)
    rows = np.array([[1, 31], [0, 0], [1, 7]])
    os_, ls_ = oracle.attn_fwd(q[rows[:, 0], rows[:, 1]], kv, c, idx[rows[:, 0], rows[:, 1]], sink,
                               0.4, 5, 4, rows)
    np.testing.assert_array_equal(os_, o[rows[:, 0], rows[:, 1]])
    np.testing.assert_array_equal(ls_, lse[rows[:, 0], rows[:, 1]])


# ------------------------------------------------------------ packed documents
def _docs(b, S, r, bounds_per_batch):
    """doc ids [b, S] from segment start positions (multiples of the ratio)."""
    doc = np.zeros((b, S), dtype=np.int32)
    for bi, starts in enumerate(bounds_per_batch):
        for k, s0 in enumerate(starts):
            doc[bi, s0:] = k + 10 * bi
    return doc


def _doc_attn(q, kv, c, idx, sink, scale, W, r, doc, do=None):
    b, S = q.shape[:2]
    rows = oracle.all_rows(b, S)
    qr = q.reshape(b * S, *q.shape[2:])
    ir = None if idx is None else idx.reshape(b * S, -1)
    o, lse = oracle.attn_fwd(qr, kv, c, ir, sink, scale, W, r, rows, doc=doc)
    if do is None:
        return o.reshape(q.shape), lse.reshape(b, S, -1)
    g = oracle.attn_bwd(qr, kv, c, ir, sink, scale, W, r, rows, do.reshape(b * S, *do.shape[2:]), doc=doc)
    return o.reshape(q.shape), lse.reshape(b, S, -1), g


@pytest.mark.parametrize("dense", [False, True])
def test_docs_attention_matches_dense_formulation(dense):
    b, S, r, W = 2, 40, 4, 7
    q, kv, c, idx, sink = _attn_case(b=b, S=S, r=r, W=W, kp=5, seed_idx=not dense)
    doc = _docs(b, S, r, [[0, 13, 28], [0, 21]])       # starts need not be block-aligned
    do = rnd(*q.shape)
    o, lse, (dq, dkv, dc, ds) = _doc_attn(q, kv, c, idx, sink, 0.3, W, r, doc, do)
    ob, lseb, _, _ = brute.attn_fwd(q, kv, c, idx, sink, 0.3, W, r, doc)
    dqb, dkvb, dcb, dsb = brute.attn_bwd(q, kv, c, idx, sink, 0.3, W, r, do, doc)
    for a, e in [(o, ob), (lse, lseb), (dq.reshape(q.shape), dqb), (dkv, dkvb), (dc, dcb), (ds, dsb)]:
        np.testing.assert_allclose(a, e, rtol=1e-11, atol=1e-11)


def test_docs_indexer_matches_dense_formulation_and_never_crosses():
    b, S, r, HI, DI, K = 2, 48, 4, 3, 5, 6
    q_i, k_i, w = rnd(b, S, HI, DI), rnd(b, S // r, DI), rnd(b, S, HI)
    doc = _docs(b, S, r, [[0, 17, 36], [0, 9]])
    idx, sc, dense = oracle.index_topk(q_i, k_i, w, r, K, doc=doc)
    Ib = brute.index_scores(q_i, k_i, w, r, doc)
    np.testing.assert_allclose(dense.reshape(b, S, -1), Ib, rtol=1e-12, atol=1e-12)
    idxb, _ = brute.topk(Ib, r, K, doc)
    np.testing.assert_array_equal(idx.reshape(b, S, -1), idxb)
    ii = idx.reshape(b, S, -1)
    for bi in range(b):
        for t in range(S):
            for j in ii[bi, t]:
                if j >= 0:
                    assert doc[bi, j * r] == doc[bi, t] and j < (t + 1) // r


def test_docs_segment_equals_standalone_sequence():
    # A document packed after another gives exactly what the method gives on
    # that document alone (positions re-based): the document rule reduces the
    # packed case to the already pinned single-sequence case.
    S, r, W, H, D, s0 = 48, 4, 9, 2, 5, 20
    q, kv, c, _, sink = _attn_case(b=1, S=S, r=r, W=W, H=H, D=D, seed_idx=False)
    doc = _docs(1, S, r, [[0, s0]])
    o, lse = _doc_attn(q, kv, c, None, sink, 0.5, W, r, doc)
    o2, lse2 = _doc_attn(q[:, s0:], kv[:, s0:], c[:, s0 // r:], None, sink, 0.5, W, r, None)
    np.testing.assert_allclose(o[:, s0:], o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[:, s0:], lse2, rtol=1e-13, atol=1e-13)
    HI, DI, K = 3, 4, 5
    q_i, k_i, w = rnd(1, S, HI, DI), rnd(1, S // r, DI), rnd(1, S, HI)
    idx, sc, _ = oracle.index_topk(q_i, k_i, w, r, K, doc=doc)
    idx2, sc2, _ = oracle.index_topk(q_i[:, s0:], k_i[:, s0 // r:], w[:, s0:], r, K)
    ii = idx.reshape(1, S, -1)[0, s0:]
    shifted = np.where(ii >= 0, ii - s0 // r, -1)
    np.testing.assert_array_equal(shifted, idx2.reshape(S - s0, -1))
    np.testing.assert_allclose(sc.reshape(1, S, -1)[0, s0:], sc2.reshape(S - s0, -1), rtol=1e-13, atol=1e-13)


def test_docs_isolation_perturbing_one_document():
    b, S, r, W = 1, 40, 4, 6
    q, kv, c, idx, sink = _attn_case(b=b, S=S, r=r, W=W, seed_idx=False)
    doc = _docs(b, S, r, [[0, 16]])
    do = rnd(*q.shape)
    o, lse, (dq, dkv, dc, _) = _doc_attn(q, kv, c, None, sink, 0.3, W, r, doc, do)
    kv2, c2, q2 = kv.copy(), c.copy(), q.copy()
    kv2[:, :16] += rnd(1, 16, kv.shape[2])
    c2[:, :4] += rnd(1, 4, c.shape[2])
    q2[:, :16] += rnd(1, 16, *q.shape[2:])
    o2, lse2, (dq2, dkv2, dc2, _) = _doc_attn(q2, kv2, c2, None, sink, 0.3, W, r, doc, do)
    np.testing.assert_array_equal(o[:, 16:], o2[:, 16:])
    np.testing.assert_array_equal(lse[:, 16:], lse2[:, 16:])
    np.testing.assert_array_equal(dq.reshape(q.shape)[:, 16:], dq2.reshape(q.shape)[:, 16:])
    np.testing.assert_array_equal(dkv[:, 16:], dkv2[:, 16:])
    np.testing.assert_array_equal(dc[:, 4:], dc2[:, 4:])


def test_docs_single_document_is_the_plain_method():
    q, kv, c, idx, sink = _attn_case()
    b, S = q.shape[:2]
    doc = np.full((b, S), 7, dtype=np.int32)
    o, lse = _doc_attn(q, kv, c, idx, sink, 0.4, 5, 4, doc)
    o2, lse2 = _fwd(q, kv, c, idx, sink, 0.4, 5, 4)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
