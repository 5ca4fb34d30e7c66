"""Pins of the simplified-DSA-over-GQA oracle (``oracle/dsa_gqa.py``).

Attention over the selected keys is tied to torch's scaled dot-product
attention with a boolean mask built from the selection (keys and values
repeated per group) and to torch autograd for the gradients; a full
selection is plain causal attention; the indexer at ratio 1 with one head
and unit weights is tied to a direct ReLU score matrix and a library sort.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import dsa_gqa

RNG = np.random.default_rng(5)


def rnd(*shape, s=1.0):
    return RNG.standard_normal(shape) * s


def _case(b=2, S=24, H=6, hkv=2, dk=8, dv=5, K=5, junk=False):
    q, k, v = rnd(b, S, H, dk), rnd(b, S, hkv, dk), rnd(b, S, hkv, dv)
    q_i, k_i = rnd(b, S, 1, 7), rnd(b, S, 7)
    idx, _, _ = oracle.index_topk(q_i, k_i, np.ones((b, S, 1)), 1, K)
    idx = idx.reshape(b, S, -1)
    if junk:
        idx = idx.copy()
        idx[:, ::3, 1] = idx[:, ::3, 0]            # repeated entry
        idx[:, 5, :] = -1                          # no valid slot
        idx[:, 7, 2] = 9                           # not yet valid
    return q, k, v, idx


def _sdpa(q, k, v, idx, scale):
    b, S, H, dk = q.shape
    hkv = k.shape[2]
    mult = np.zeros((b, S, S))
    for bi in range(b):
        for t in range(S):
            for j in idx[bi, t]:
                if 0 <= j <= t:
                    mult[bi, t, j] += 1
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(H // hkv, dim=2).transpose(1, 2)   # [b,H,S,dk]
    vv = tv.repeat_interleave(H // hkv, dim=2).transpose(1, 2)
    logits = scale * tq.transpose(1, 2) @ kk.transpose(-1, -2)    # [b,H,S,S]
    m = torch.tensor(mult)[:, None]
    # a key selected n times enters the softmax n times: log n added to its logit
    logits = torch.where(m > 0, logits + torch.log(m.clamp(min=1)), torch.full_like(logits, -np.inf))
    lse = torch.logsumexp(logits, dim=-1)
    p = torch.where(m > 0, torch.exp(logits - lse[..., None]), torch.zeros_like(logits))
    out = (p @ vv).transpose(1, 2)
    return tq, tk, tv, out, lse.transpose(1, 2)


@pytest.mark.parametrize("junk", [False, True])
def test_against_masked_attention_and_autograd(junk):
    q, k, v, idx = _case(junk=junk)
    scale = 0.35
    o, lse = dsa_gqa.fwd(q, k, v, idx, scale)
    tq, tk, tv, to, tlse = _sdpa(q, k, v, idx, scale)
    ref_o = to.detach().numpy()
    ref_lse = tlse.detach().numpy()
    empty = np.isneginf(lse)
    assert np.array_equal(empty, np.isneginf(ref_lse)) and (empty.any() == junk)
    np.testing.assert_allclose(o[~empty], ref_o[~empty], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o[empty], 0.0)
    np.testing.assert_allclose(lse[~empty], ref_lse[~empty], rtol=1e-12, atol=1e-13)
    do = rnd(*o.shape)
    dq, dk, dv = dsa_gqa.bwd(q, k, v, idx, scale, o, lse, do)
    sel = torch.tensor(~empty)[..., None]
    (torch.where(sel, to, torch.zeros_like(to)) * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_full_selection_is_causal_attention():
    b, S, H, hkv, d = 1, 12, 4, 2, 8
    q, k, v = rnd(b, S, H, d), rnd(b, S, hkv, d), rnd(b, S, hkv, d)
    idx = np.tile(np.arange(S), (b, S, 1)).astype(np.int32)       # every earlier key (later ones invalid)
    o, _ = dsa_gqa.fwd(q, k, v, idx, 0.5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q).transpose(1, 2), torch.tensor(k).repeat_interleave(2, 2).transpose(1, 2),
        torch.tensor(v).repeat_interleave(2, 2).transpose(1, 2), is_causal=True, scale=0.5).transpose(1, 2)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_single_selected_key_copies_its_value():
    q, k, v, _ = _case(K=1)
    idx = np.zeros((2, 24, 1), dtype=np.int32)       # key 0 for everyone
    o, lse = dsa_gqa.fwd(q, k, v, idx, 0.3)
    for h in range(6):
        np.testing.assert_allclose(o[:, :, h], v[:, 0:1, h // 3].repeat(24, axis=1), rtol=1e-14)
        np.testing.assert_allclose(lse[:, :, h], 0.3 * np.einsum("btd,bd->bt", q[:, :, h], k[:, 0, h // 3]),
                                   rtol=1e-13)


def test_simplified_indexer_is_relu_scores_and_library_topk():
    b, S, K = 1, 30, 6
    q_i, k_i = rnd(b, S, 1, 7), rnd(b, S, 7)
    idx, sc, _ = oracle.index_topk(q_i, k_i, np.ones((b, S, 1)), 1, K)
    scores = np.maximum(np.einsum("bsd,bjd->bsj", q_i[:, :, 0], k_i), 0.0)[0]
    for t in range(S):
        cand = np.arange(t + 1)
        order = np.lexsort((cand, -(scores[t, cand] + 0.0)))[:K]
        np.testing.assert_array_equal(idx[t, :min(K, t + 1)], np.sort(cand[order]))
