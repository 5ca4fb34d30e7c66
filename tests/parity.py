"""Helpers for GPU-vs-oracle parity tests.

Bars (stated for the method): floating-point outputs satisfy
max|gpu - ref| <= tol * max|ref| with tol = 1e-2 for bf16 inputs and 1e-5
for fp32 inputs, per output tensor.  Top-k index sets are bit-exact outside a
near-tie band: with s* the oracle's K'-th score of a row, entries with
|I_j - s*| < 1e-4 may differ; everything else (the set outside the band, the
count, the -1 padding, ascending order) must match exactly.  Rows with
n_valid <= K' must match exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

BAND = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol_of(dtype) -> float:
    return 1e-2 if dtype == torch.bfloat16 else 1e-5


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def check_close(name, got, ref, tol):
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.abs(got - ref).max())
    bound = tol * float(np.abs(ref).max())
    say(f"  {name}: max|err| = {err:.3e}  bound = {bound:.3e}")
    assert err <= bound, f"{name}: max|err| {err:.3e} > {tol:g} * max|ref| = {bound:.3e}"
    return err


def n_valid(t, ratio, nc):
    return np.minimum((np.asarray(t) + 1) // ratio, nc)


def check_topk_rows(gpu_idx, gpu_score, ora_idx, ora_dense, rows_t, ratio, nc, kp, score_tol, docs=False):
    """gpu_idx/gpu_score/ora_idx: [n, K']; ora_dense: [n, n_c] oracle scores.

    Without documents the selectable blocks of row t are 0..n_valid(t)-1; with
    ``docs`` they are the blocks the oracle scored (finite entries of its row),
    which is how the oracle marks the blocks of the query's own document."""
    gpu_idx = np.asarray(gpu_idx)
    ora_idx = np.asarray(ora_idx)
    exact_rows = 0
    mism = []
    smax = np.abs(ora_dense[np.isfinite(ora_dense)]).max() if np.isfinite(ora_dense).any() else 1.0
    for n, t in enumerate(rows_t):
        nv = int(n_valid(t, ratio, nc))
        valid = np.nonzero(np.isfinite(ora_dense[n]))[0] if docs else np.arange(nv)
        if not docs:
            assert np.array_equal(valid, np.nonzero(np.isfinite(ora_dense[n]))[0])
        m = min(kp, len(valid))
        g, o = gpu_idx[n], ora_idx[n]
        assert np.all(g[m:] == -1), f"row t={t}: expected {kp - m} trailing -1, got {g}"
        gs = g[:m]
        assert np.all(np.isin(gs, valid)), f"row t={t}: index outside the selectable blocks"
        assert np.all(np.diff(gs) > 0), f"row t={t}: not strictly ascending"
        if gpu_score is not None:
            sc = np.asarray(gpu_score[n])
            assert np.all(np.isneginf(sc[m:]))
            err = np.abs(sc[:m] - ora_dense[n, gs]).max() if m else 0.0
            assert err <= score_tol * smax, f"row t={t}: score error {err} > {score_tol * smax}"
        if len(valid) <= kp:
            np.testing.assert_array_equal(gs, valid)
            exact_rows += 1
            continue
        sstar = np.min(ora_dense[n, o[:m]])          # the oracle's K'-th score
        band = set(valid[np.abs(ora_dense[n, valid] - sstar) < BAND].tolist())
        gset = set(gs.tolist()) - band
        oset = set(o[:m].tolist()) - band
        if gset != oset:
            mism.append((t, sorted(gset - oset)[:5], sorted(oset - gset)[:5]))
        else:
            exact_rows += 1 if set(gs.tolist()) == set(o[:m].tolist()) else 0
    assert not mism, f"top-k mismatch outside the near-tie band in {len(mism)} rows, e.g. {mism[:3]}"
    return exact_rows


def oracle_inputs(inp, keys):
    return {k: (None if inp.get(k) is None else f64(inp[k])) for k in keys}


def sample_rows(b, S, n, seed, must=()):
    rng = np.random.default_rng(seed)
    rows = set()
    for t in must:
        for bi in range(b):
            if 0 <= t < S:
                rows.add((bi, t))
    while len(rows) < min(n, b * S):
        rows.add((int(rng.integers(b)), int(rng.integers(S))))
    return np.array(sorted(rows), dtype=np.int64)
