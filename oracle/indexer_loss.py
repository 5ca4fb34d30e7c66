"""fp64 oracle of the indexer's training path (the distillation loss).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): imported by ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` only.

What is computed, per query row t with its selected index row (the slots
whose block j satisfies 0 <= j < min((t+1)//ratio, n_c) are its support):

* Teacher (torchtitan PR #4452, description of the lightning indexer and the
  indexer distillation loss; Megatron-LM PR #6400, thread on the teacher's
  normalisation): the mass of slot s is the sum over attention heads h of
  exp(scale * <q[t,h], c[j_s]> - LSE[t,h]), where LSE is the attention
  forward's per-head log-sum-exp over window rows, selected compressed rows
  and the sink.  The target is that mass L1-normalised over the support; a
  row with an empty support has an all-zero target.  The same PR #6400 thread
  gives the equivalent per-head form sigmoid(lse_c - lse_nc) * softmax_h;
  the tests pin the two against each other.  The teacher is detached.
* Student (PR #4452, second differentiable pass over the selected entries;
  Megatron-LM PR #7152, commit on reusing the routing scores): the selected
  indexer scores I[t,s] = sum_h w[t,h] * ReLU(<q_i[t,h], k_i[j_s]>) and their
  softmax over the support.
* Loss: KL(target || predict) = sum over the support of
  target * (log target - log predict) (0 where target is 0), one value per
  row.
* Gradient (PR #6400 thread: predict * sum(target) - target, which is zero on
  a zero-mass row): dI[t,s] = dkl[t] * (predict * sum(target) - target),
  then through the student: dw[t,h] = sum_s dI * ReLU(a), dq_i[t,h] =
  sum_s dI * w * [a > 0] * k_i[j_s], and dk_i[j] += the same coefficient times
  q_i[t,h], accumulated over every (row, slot) that selected j (a block
  selected by many queries sums all their terms; a repeated index in one row
  counts once per slot).  a = <q_i[t,h], k_i[j_s]>; the ReLU's derivative at
  0 is taken as 0.

Dense warm-up form (Megatron-LM PR #7152, the commit adding the dense
warm-up tile plan: the dense teacher scores every attention head against
the same keys, the indexer against all of them): the support of row t is
every valid block j < min((t+1)//ratio, n_c) instead of the selected slots;
teacher, student, KL and gradients are the ones above over that support
(``dense_warmup_loss``).  Written over dense per-row matrices, not through
the slot functions above.

Plain NumPy, one query row at a time; library matmuls and exp/log only.
"""
from __future__ import annotations

import numpy as np


def _support(idx_row, t, ratio, nc):
    nv = min((int(t) + 1) // ratio, nc)
    idx_row = np.asarray(idx_row, dtype=np.int64)
    return np.nonzero((idx_row >= 0) & (idx_row < nv))[0]


def _logsumexp(x, axis):
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def teacher_target(q_rows, c, lse_rows, idx_rows, scale, ratio, rows):
    """Target distribution over the slots of each listed row.

    q_rows [n,H,D], lse_rows [n,H] (the attention forward's LSE of those
    rows), c [b,n_c,D], idx_rows [n,K'], rows [n,2] (batch, t).
    Returns target [n,K'] (0 outside the support)."""
    q = np.asarray(q_rows, np.float64)
    c = np.asarray(c, np.float64)
    lse = np.asarray(lse_rows, np.float64)
    idx = np.asarray(idx_rows)
    n, kp = idx.shape
    nc = c.shape[1]
    target = np.zeros((n, kp))
    for r in range(n):
        b, t = int(rows[r, 0]), int(rows[r, 1])
        sup = _support(idx[r], t, ratio, nc)
        if len(sup) == 0:
            continue
        logits = scale * (q[r] @ c[b, idx[r, sup]].T)             # [H, |sup|]
        log_mass = _logsumexp(logits - lse[r][:, None], axis=0)   # log sum_h exp(l - LSE_h)
        target[r, sup] = np.exp(log_mass - _logsumexp(log_mass, axis=0))
    return target


def selected_scores(q_i_rows, k_i, w_rows, idx_rows, ratio, rows):
    """Student logits I[n,K'] over each row's slots (-inf outside the support)."""
    q = np.asarray(q_i_rows, np.float64)
    k = np.asarray(k_i, np.float64)
    w = np.asarray(w_rows, np.float64)
    idx = np.asarray(idx_rows)
    n, kp = idx.shape
    nc = k.shape[1]
    out = np.full((n, kp), -np.inf)
    for r in range(n):
        b, t = int(rows[r, 0]), int(rows[r, 1])
        sup = _support(idx[r], t, ratio, nc)
        if len(sup) == 0:
            continue
        a = q[r] @ k[b, idx[r, sup]].T                            # [HI, |sup|]
        out[r, sup] = w[r] @ np.maximum(a, 0.0)
    return out


def kl_loss(target, scores):
    """Per-row KL(target || softmax(scores)) over the finite entries of scores.

    Returns (kl [n], predict [n,K'])."""
    target = np.asarray(target, np.float64)
    s = np.asarray(scores, np.float64)
    n, kp = s.shape
    kl = np.zeros(n)
    predict = np.zeros((n, kp))
    for r in range(n):
        sup = np.nonzero(np.isfinite(s[r]))[0]
        if len(sup) == 0:
            continue
        logp = s[r, sup] - _logsumexp(s[r, sup], axis=0)
        predict[r, sup] = np.exp(logp)
        tr = target[r, sup]
        pos = tr > 0
        kl[r] = np.sum(tr[pos] * (np.log(tr[pos]) - logp[pos]))
    return kl, predict


def loss_bwd(q_i_rows, k_i, w_rows, idx_rows, ratio, rows, target, predict, dkl):
    """Gradients of sum_t dkl[t] * KL_t with respect to the student's inputs.

    Returns (dq_i [n,HI,DI], dw [n,HI], dk_i [b,n_c,DI], dI [n,K'])."""
    q = np.asarray(q_i_rows, np.float64)
    k = np.asarray(k_i, np.float64)
    w = np.asarray(w_rows, np.float64)
    idx = np.asarray(idx_rows)
    target = np.asarray(target, np.float64)
    predict = np.asarray(predict, np.float64)
    dkl = np.asarray(dkl, np.float64)
    n, kp = idx.shape
    b_all, nc, di = k.shape
    dq = np.zeros_like(q)
    dw = np.zeros_like(w)
    dk = np.zeros_like(k)
    dI = np.zeros((n, kp))
    for r in range(n):
        b, t = int(rows[r, 0]), int(rows[r, 1])
        sup = _support(idx[r], t, ratio, nc)
        if len(sup) == 0:
            continue
        g = dkl[r] * (predict[r, sup] * target[r, sup].sum() - target[r, sup])
        dI[r, sup] = g
        js = idx[r, sup]
        a = q[r] @ k[b, js].T                                     # [HI, |sup|]
        dw[r] = np.maximum(a, 0.0) @ g
        coef = w[r][:, None] * (a > 0) * g[None, :]               # dI * w * ReLU'(a)
        dq[r] = coef @ k[b, js]
        np.add.at(dk[b], js, coef.T @ q[r])
    return dq, dw, dk, dI


def indexer_loss(q_rows, c, lse_rows, q_i_rows, k_i, w_rows, idx_rows, scale, ratio, rows, dkl=None):
    """The whole path for listed rows.

    Returns a dict with target, scores, predict, kl and, when ``dkl`` is
    given, dq_i, dw, dk_i and dI."""
    target = teacher_target(q_rows, c, lse_rows, idx_rows, scale, ratio, rows)
    scores = selected_scores(q_i_rows, k_i, w_rows, idx_rows, ratio, rows)
    kl, predict = kl_loss(target, scores)
    out = dict(target=target, scores=scores, predict=predict, kl=kl)
    if dkl is not None:
        dq, dw, dk, dI = loss_bwd(q_i_rows, k_i, w_rows, idx_rows, ratio, rows, target, predict, dkl)
        out.update(dq_i=dq, dw=dw, dk_i=dk, dI=dI)
    return out


def dense_warmup_loss(q_rows, c, lse_rows, q_i_rows, k_i, w_rows, scale, ratio, rows, dkl=None):
    """Dense warm-up loss over every valid block of each listed row.

    q_rows [n,H,D], c [b,n_c,D], lse_rows [n,H], q_i_rows [n,HI,DI],
    k_i [b,n_c,DI], w_rows [n,HI], rows [n,2] (batch, t), dkl [n] or None.
    Returns a dict with target [n,n_c], scores [n,n_c] (-inf past n_valid),
    predict [n,n_c], kl [n] and, with ``dkl``, dq_i, dw, dk_i and dI [n,n_c]."""
    q = np.asarray(q_rows, np.float64)
    c = np.asarray(c, np.float64)
    lse = np.asarray(lse_rows, np.float64)
    qi = np.asarray(q_i_rows, np.float64)
    k = np.asarray(k_i, np.float64)
    w = np.asarray(w_rows, np.float64)
    n = q.shape[0]
    nc = c.shape[1]
    target = np.zeros((n, nc))
    scores = np.full((n, nc), -np.inf)
    predict = np.zeros((n, nc))
    kl = np.zeros(n)
    grads = dkl is not None
    if grads:
        dkl = np.asarray(dkl, np.float64)
        dq, dw, dk, dI = np.zeros_like(qi), np.zeros_like(w), np.zeros_like(k), np.zeros((n, nc))
    for r in range(n):
        b, t = int(rows[r, 0]), int(rows[r, 1])
        nv = min((t + 1) // ratio, nc)
        if nv == 0:
            continue
        # teacher: log of the head-summed probability mass of each block
        logits = scale * (q[r] @ c[b, :nv].T)                     # [H, nv]
        log_mass = _logsumexp(logits - lse[r][:, None], axis=0)   # [nv]
        tg = np.exp(log_mass - _logsumexp(log_mass, axis=0))
        target[r, :nv] = tg
        # student: weighted ReLU scores of the indexer and their softmax
        a = qi[r] @ k[b, :nv].T                                   # [HI, nv]
        I = w[r] @ np.maximum(a, 0.0)
        scores[r, :nv] = I
        logp = I - _logsumexp(I, axis=0)
        predict[r, :nv] = np.exp(logp)
        pos = tg > 0
        kl[r] = np.sum(tg[pos] * (np.log(tg[pos]) - logp[pos]))
        if grads:
            g = dkl[r] * (predict[r, :nv] * tg.sum() - tg)
            dI[r, :nv] = g
            dw[r] = np.maximum(a, 0.0) @ g
            coef = w[r][:, None] * (a > 0) * g[None, :]           # [HI, nv]
            dq[r] = coef @ k[b, :nv]
            dk[b, :nv] += coef.T @ qi[r]
    out = dict(target=target, scores=scores, predict=predict, kl=kl)
    if grads:
        out.update(dq_i=dq, dw=dw, dk_i=dk, dI=dI)
    return out
