"""Pins of the dense warm-up form of the indexer loss
(``oracle.indexer_loss.dense_warmup_loss``).

It is tied to the selected-block form run with index rows that list every
block (a different code path over slots), to torch autograd over a dense
torch formulation with torch's own KL divergence, and to closed forms: with
one head and an LSE over the compressed blocks alone the teacher is the
attention softmax itself; rows before the first block are empty.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import indexer_loss as il

RNG = np.random.default_rng(91)


def rnd(*shape, s=1.0):
    return RNG.standard_normal(shape) * s


def _case(b=2, S=37, H=3, D=6, HI=2, DI=5, r=4, W=5):
    nc = S // r
    q, kv, c = rnd(b, S, H, D), rnd(b, S, D), rnd(b, nc, D)
    sink = rnd(H)
    q_i, k_i, w = rnd(b, S, HI, DI), rnd(b, nc, DI), rnd(b, S, HI, s=0.5)
    rows = oracle.all_rows(b, S)
    scale = 0.4
    # the warm-up's attention attends every valid block (dense mode)
    _, lse = oracle.attn_fwd(q.reshape(b * S, H, D), kv, c, None, sink, scale, W, r, rows)
    return dict(q=q.reshape(b * S, H, D), c=c, q_i=q_i.reshape(b * S, HI, DI), k_i=k_i, w=w.reshape(b * S, HI),
                rows=rows, lse=lse, scale=scale, r=r, nc=nc)


def test_dense_equals_selected_form_with_every_block_listed():
    k = _case()
    n = len(k["rows"])
    full = np.tile(np.arange(k["nc"], dtype=np.int32), (n, 1))
    dkl = rnd(n)
    sp = il.indexer_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], full, k["scale"], k["r"], k["rows"],
                         dkl=dkl)
    de = il.dense_warmup_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], k["scale"], k["r"], k["rows"],
                              dkl=dkl)
    np.testing.assert_allclose(de["target"], sp["target"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(de["kl"], sp["kl"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(de["dI"], sp["dI"], rtol=1e-12, atol=1e-14)
    for g in ("dq_i", "dw", "dk_i"):
        np.testing.assert_allclose(de[g], sp[g], rtol=1e-11, atol=1e-13)
    assert np.array_equal(np.isfinite(de["scores"]), np.isfinite(sp["scores"]))


def test_dense_loss_and_gradients_against_torch_autograd():
    k = _case(b=1, S=41, H=2, HI=3)
    n = len(k["rows"])
    dkl = rnd(n)
    got = il.dense_warmup_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], k["scale"], k["r"], k["rows"],
                               dkl=dkl)
    qi = torch.tensor(k["q_i"], requires_grad=True)
    ki = torch.tensor(k["k_i"], requires_grad=True)
    w = torch.tensor(k["w"], requires_grad=True)
    q, c, lse = torch.tensor(k["q"]), torch.tensor(k["c"]), torch.tensor(k["lse"])
    total = torch.zeros((), dtype=torch.float64)
    kls = []
    for m, (b, t) in enumerate(k["rows"]):
        nv = min((t + 1) // k["r"], k["nc"])
        if nv == 0:
            kls.append(0.0)
            continue
        with torch.no_grad():                              # the teacher is detached
            probs = torch.exp(k["scale"] * q[m] @ c[b, :nv].T - lse[m][:, None])   # [H, nv]
            mass = probs.sum(0)
            target = mass / mass.sum()
        logits = (w[m][:, None] * torch.relu(qi[m] @ ki[b, :nv].T)).sum(0)
        kl = torch.nn.functional.kl_div(torch.log_softmax(logits, dim=0), target, reduction="sum")
        kls.append(kl.item())
        total = total + float(dkl[m]) * kl
    total.backward()
    np.testing.assert_allclose(got["kl"], kls, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got["dq_i"], qi.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(got["dw"], w.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(got["dk_i"], ki.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_one_head_teacher_is_the_softmax_over_blocks():
    # one head whose LSE runs over the compressed blocks only: the teacher is
    # that head's attention softmax over the blocks (any LSE shift cancels)
    b, S, D, r = 1, 30, 4, 3
    nc = S // r
    q, c = rnd(S, 1, D), rnd(b, nc, D)
    rows = oracle.all_rows(b, S)
    scale = 0.7
    lse = np.zeros((S, 1))
    for t in range(S):
        nv = min((t + 1) // r, nc)
        if nv:
            l = scale * q[t, 0] @ c[0, :nv].T
            lse[t, 0] = np.log(np.exp(l).sum()) + 3.0
    out = il.dense_warmup_loss(q, c, lse, rnd(S, 1, 2), rnd(b, nc, 2), rnd(S, 1), scale, r, rows)
    for t in range(S):
        nv = min((t + 1) // r, nc)
        if nv == 0:
            assert np.all(out["target"][t] == 0) and out["kl"][t] == 0
            continue
        l = scale * q[t, 0] @ c[0, :nv].T
        sm = np.exp(l - l.max())
        np.testing.assert_allclose(out["target"][t, :nv], sm / sm.sum(), rtol=1e-13)
        assert np.all(out["target"][t, nv:] == 0)


def test_kl_nonnegative_di_rows_sum_to_zero_and_one_block_rows_vanish():
    k = _case(b=1, S=24)
    out = il.dense_warmup_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], k["scale"], k["r"], k["rows"],
                               dkl=np.ones(24))
    assert np.all(out["kl"] >= -1e-14)
    # dI sums to zero on every row with mass (softmax minus a distribution)
    np.testing.assert_allclose(out["dI"].sum(axis=1), 0.0, atol=1e-13)
    # a one-block row: target and student are both 1 on it, KL and gradients vanish
    t1 = [m for m, (_, t) in enumerate(k["rows"]) if (t + 1) // k["r"] == 1]
    assert t1
    for m in t1:
        assert out["kl"][m] == pytest.approx(0.0, abs=1e-15)
        assert np.all(out["dq_i"][m] == 0)
