"""Pins of the indexer-loss oracle (``oracle/indexer_loss.py``).

The teacher is tied to the per-head form the pages give beside it
(sigmoid(lse_c - lse_nc) times each head's softmax over the selected blocks,
with lse_nc the window + sink log-sum-exp computed by the attention oracle),
the loss and its gradients to torch autograd over torch's own KL divergence,
and both to closed forms and invariants (empty and single-slot rows, a
zero-loss student, logits near 1000 that overflow a naive exponential).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from oracle import indexer_loss as il

RNG = np.random.default_rng(77)


def rnd(*shape, s=1.0):
    return RNG.standard_normal(shape) * s


def _case(b=2, S=40, H=3, D=6, HI=2, DI=5, r=4, W=5, K=4, dup=False):
    nc = S // r
    q, kv, c = rnd(b, S, H, D), rnd(b, S, D), rnd(b, nc, D)
    sink = rnd(H)
    q_i, k_i, w = rnd(b, S, HI, DI), rnd(b, nc, DI), rnd(b, S, HI, s=0.5)
    idx, score, _ = oracle.index_topk(q_i, k_i, w, r, K)
    idx = idx.reshape(b * S, -1)
    if dup:
        # repeat a valid entry in some rows (never produced by the indexer;
        # the loss then counts it once per slot)
        for n in range(b * S):
            if idx[n, 1] >= 0:
                idx[n, 1] = idx[n, 0]
    rows = oracle.all_rows(b, S)
    scale = 0.4
    _, lse = oracle.attn_fwd(q.reshape(b * S, H, D), kv, c, idx, sink, scale, W, r, rows)
    return dict(q=q.reshape(b * S, H, D), kv=kv, c=c, sink=sink, q_i=q_i.reshape(b * S, HI, DI), k_i=k_i,
                w=w.reshape(b * S, HI), idx=idx, rows=rows, lse=lse, scale=scale, r=r, W=W)


def test_teacher_equals_per_head_sigmoid_form():
    k = _case()
    target = il.teacher_target(k["q"], k["c"], k["lse"], k["idx"], k["scale"], k["r"], k["rows"])
    # window + sink LSE from the attention oracle with no compressed slot
    none = np.full_like(k["idx"], -1)
    _, lse_nc = oracle.attn_fwd(k["q"], k["kv"], k["c"], none, k["sink"], k["scale"], k["W"], k["r"], k["rows"])
    nc = k["c"].shape[1]
    checked = 0
    for n, (b, t) in enumerate(k["rows"]):
        nv = min((t + 1) // k["r"], nc)
        sup = [s for s in range(k["idx"].shape[1]) if 0 <= k["idx"][n, s] < nv]
        if not sup:
            assert np.all(target[n] == 0)
            continue
        ell = k["scale"] * k["q"][n] @ k["c"][b, k["idx"][n, sup]].T           # [H, |sup|]
        lse_c = np.log(np.exp(ell).sum(axis=1))
        m = 1.0 / (1.0 + np.exp(-(lse_c - lse_nc[n])))                         # compressed mass per head
        probs = np.exp(ell) / np.exp(ell).sum(axis=1, keepdims=True) * m[:, None]
        ref = probs.sum(axis=0)
        np.testing.assert_allclose(target[n, sup], ref / ref.sum(), rtol=1e-12, atol=1e-15)
        assert np.all(np.delete(target[n], sup) == 0)
        checked += 1
    assert checked > 40


def test_teacher_lse_is_the_attention_lse():
    # the LSE the teacher consumes is the one both attention formulations give
    k = _case(b=1, S=24)
    _, lse_b, _, _ = brute.attn_fwd(k["q"].reshape(1, 24, 3, 6), k["kv"], k["c"], k["idx"].reshape(1, 24, -1),
                              k["sink"], k["scale"], k["W"], k["r"])
    np.testing.assert_allclose(k["lse"], lse_b.reshape(24, 3), rtol=1e-13)


@pytest.mark.parametrize("dup", [False, True])
def test_loss_and_gradients_against_torch_autograd(dup):
    k = _case(dup=dup)
    target = il.teacher_target(k["q"], k["c"], k["lse"], k["idx"], k["scale"], k["r"], k["rows"])
    dkl = rnd(len(k["rows"]))
    got = il.indexer_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], k["idx"], k["scale"], k["r"],
                          k["rows"], dkl=dkl)
    qi = torch.tensor(k["q_i"], requires_grad=True)
    ki = torch.tensor(k["k_i"], requires_grad=True)
    w = torch.tensor(k["w"], requires_grad=True)
    nc = k["k_i"].shape[1]
    total = 0
    kls = []
    for n, (b, t) in enumerate(k["rows"]):
        nv = min((t + 1) // k["r"], nc)
        sup = [s for s in range(k["idx"].shape[1]) if 0 <= k["idx"][n, s] < nv]
        if not sup:
            kls.append(0.0)
            continue
        js = torch.tensor(k["idx"][n, sup], dtype=torch.long)
        a = qi[n] @ ki[b, js].T
        logits = (w[n][:, None] * torch.relu(a)).sum(0)
        logp = torch.log_softmax(logits, dim=0)
        kl = torch.nn.functional.kl_div(logp, torch.tensor(target[n, sup]), reduction="sum")
        kls.append(kl.item())
        total = total + float(dkl[n]) * kl
    total.backward()
    np.testing.assert_allclose(got["kl"], kls, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got["dq_i"], qi.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got["dw"], w.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got["dk_i"], ki.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_selected_scores_equal_the_indexer_scores():
    # the student's logits on the selected slots are the routing scores
    k = _case()
    I = il.selected_scores(k["q_i"], k["k_i"], k["w"], k["idx"], k["r"], k["rows"])
    dense = oracle.index_scores(k["q_i"], k["k_i"], k["w"], k["r"], k["rows"])
    for n in range(len(k["rows"])):
        for s, j in enumerate(k["idx"][n]):
            if j >= 0:
                assert I[n, s] == pytest.approx(dense[n, j], rel=1e-13, abs=1e-14)
            else:
                assert I[n, s] == -np.inf


def test_large_logits_two_heads_two_keys():
    # logits near 1000 overflow exp() in any precision; the target only
    # depends on logit - LSE per head, given here in closed form
    q = np.array([[[1000.0], [998.0]]])          # [n=1, H=2, D=1]
    c = np.array([[[1.0], [0.999]]])             # blocks 0, 1
    lse = np.array([[1001.0, 1000.0]])
    idx = np.array([[0, 1]])
    rows = np.array([[0, 7]])                    # t = 7, ratio 4: both blocks valid
    x = np.array([[1000.0 - 1001.0, 999.0 - 1001.0], [998.0 - 1000.0, 998.0 * 0.999 - 1000.0]])
    mass = np.exp(x[0]) + np.exp(x[1])
    target = il.teacher_target(q, c, lse, idx, 1.0, 4, rows)
    np.testing.assert_allclose(target[0], mass / mass.sum(), rtol=1e-12)
    assert math.isclose(target.sum(), 1.0, rel_tol=1e-15)


def test_teacher_common_shift_cancels_per_head_shift_does_not():
    k = _case()
    args = (k["q"], k["c"])
    t0 = il.teacher_target(*args, k["lse"], k["idx"], k["scale"], k["r"], k["rows"])
    t1 = il.teacher_target(*args, k["lse"] + 300.0, k["idx"], k["scale"], k["r"], k["rows"])
    np.testing.assert_allclose(t1, t0, rtol=1e-11, atol=1e-15)
    shift = np.array([0.0, 2.0, -1.0])
    t2 = il.teacher_target(*args, k["lse"] + shift, k["idx"], k["scale"], k["r"], k["rows"])
    assert np.abs(t2 - t0).max() > 1e-3


def test_empty_support_rows_are_zero():
    k = _case()
    dkl = np.ones(len(k["rows"]))
    got = il.indexer_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], k["idx"], k["scale"], k["r"],
                          k["rows"], dkl=dkl)
    empty = k["rows"][:, 1] < k["r"] - 1                    # t < r - 1: no valid block yet
    assert empty.sum() == 2 * (k["r"] - 1)
    assert np.all(got["target"][empty] == 0) and np.all(got["kl"][empty] == 0)
    assert np.all(got["dq_i"][empty] == 0) and np.all(got["dw"][empty] == 0)
    # an all-padding index row behaves the same
    idx = np.full_like(k["idx"], -1)
    got = il.indexer_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], idx, k["scale"], k["r"],
                          k["rows"], dkl=dkl)
    assert np.all(got["kl"] == 0) and np.all(got["dk_i"] == 0) and np.all(got["dq_i"] == 0)


def test_single_slot_rows_have_zero_loss_and_gradient():
    k = _case(K=1)
    got = il.indexer_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], k["idx"], k["scale"], k["r"],
                          k["rows"], dkl=np.ones(len(k["rows"])))
    valid = k["idx"][:, 0] >= 0
    np.testing.assert_allclose(got["target"][valid, 0], 1.0, rtol=1e-15)
    np.testing.assert_allclose(got["predict"][valid, 0], 1.0, rtol=1e-15)
    assert np.abs(got["kl"]).max() < 1e-15
    assert np.abs(got["dI"]).max() < 1e-15
    assert np.abs(got["dk_i"]).max() < 1e-14


def test_kl_is_nonnegative_zero_for_matching_student_and_gradient_rows_sum_to_zero():
    k = _case()
    target = il.teacher_target(k["q"], k["c"], k["lse"], k["idx"], k["scale"], k["r"], k["rows"])
    scores = il.selected_scores(k["q_i"], k["k_i"], k["w"], k["idx"], k["r"], k["rows"])
    kl, predict = il.kl_loss(target, scores)
    assert np.all(kl >= -1e-15) and kl.max() > 1e-3
    # a student whose logits are log(target) + const matches the teacher
    match = np.where(target > 0, np.log(np.where(target > 0, target, 1.0)) + 3.0, -np.inf)
    kl0, p0 = il.kl_loss(target, match)
    assert np.abs(kl0).max() < 1e-13
    np.testing.assert_allclose(p0, target, rtol=1e-12, atol=1e-16)
    dq, dw, dk, dI = il.loss_bwd(k["q_i"], k["k_i"], k["w"], k["idx"], k["r"], k["rows"], target, predict,
                                 np.ones(len(k["rows"])))
    np.testing.assert_allclose(dI.sum(axis=1), 0.0, atol=1e-15)


def test_gradients_linear_in_dkl():
    k = _case()
    a = il.indexer_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], k["idx"], k["scale"], k["r"],
                        k["rows"], dkl=np.full(len(k["rows"]), 1.0))
    b = il.indexer_loss(k["q"], k["c"], k["lse"], k["q_i"], k["k_i"], k["w"], k["idx"], k["scale"], k["r"],
                        k["rows"], dkl=np.full(len(k["rows"]), -2.5))
    for key in ("dq_i", "dw", "dk_i"):
        np.testing.assert_allclose(b[key], -2.5 * a[key], rtol=1e-13, atol=1e-15)
