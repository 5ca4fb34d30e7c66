"""Golden fixtures: the pages' stated index-space constants and an oracle
regression fixture (``tests/golden/oracle_tiny.npz``, written by
``tests/golden/make_golden.py`` from the oracle alone)."""
import json
import os

import numpy as np

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _const():
    with open(os.path.join(GOLD, "page_constants.json")) as f:
        return json.load(f)


def test_page_index_space_constants():
    c = _const()["csa4_layer"]
    n_c = c["sq"] // c["ratio"]
    assert n_c == c["n_compressed"]
    assert c["sq"] + n_c == c["n_kv"]              # raw rows first, compressed rows at offset sq
    dense = c["b"] * c["sq"] * c["n_kv"] * c["head_dim"] * 2
    assert abs(dense - c["dense_grad_buffer_bytes_bf16_approx"]) / dense < 0.01
    m = _const()["causal_mask"]
    assert abs(m["sq"] * m["n_compressed"] * 4 / 2**20 - m["bytes_approx_mb"]) <= 1.0
    d = _const()["duplicate_window_logits"]
    assert abs(d["sq"] * d["window"] * d["heads"] * d["head_dim"] / 1e9 - d["gmac_approx"]) < 0.05


def test_oracle_causal_validity_matches_page_mask_rule():
    # the mask rule: block j is invalid for query t iff j >= (t+1)//ratio
    c = _const()["causal_mask"]
    S, nc = c["sq"], c["n_compressed"]
    r = S // nc
    rows = np.array([[0, t] for t in (0, 2, 3, 4, 7, 100, 2047, 4094, 4095)])
    q = np.ones((len(rows), 1, 1))
    k = np.ones((1, nc, 1))
    I = oracle.index_scores(q, k, np.ones((len(rows), 1)), r, rows)
    for (_, t), row in zip(rows, I):
        nv = int(np.isfinite(row).sum())
        assert nv == (t + 1) // r
        assert np.all(np.isfinite(row[:nv])) and np.all(np.isneginf(row[nv:]))


def test_oracle_regression_fixture():
    import sys
    sys.path.insert(0, GOLD)
    import make_golden
    got = make_golden.compute()
    ref = np.load(os.path.join(GOLD, "oracle_tiny.npz"))
    for k in ref.files:
        if ref[k].dtype.kind == "i":
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        else:
            np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-13, err_msg=k)
