"""Pins of the compressor-epilogue oracle (``oracle/epilogue.py``).

The norm is tied to torch's RMS norm, the rotation to complex multiplication
of interleaved pairs and to the relative-position property of rotary
embeddings, and the backward (through the pooling as well) to torch autograd
over an independent torch formulation of pooling + norm + rotation.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import epilogue as ep

RNG = np.random.default_rng(99)


def rnd(*shape, s=1.0):
    return RNG.standard_normal(shape) * s


def test_norm_matches_torch_rms_norm():
    c, w = rnd(2, 9, 16), rnd(16)
    got = ep.epilogue(c, w, 1e-6, 0, 40000.0)
    ref = torch.nn.functional.rms_norm(torch.tensor(c), (16,), torch.tensor(w), eps=1e-6).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("rope_dim", [16, 8, 2])
def test_rotation_is_complex_multiplication(rope_dim):
    c = rnd(2, 11, 16)
    got = ep.epilogue(c, None, 0.0, rope_dim, 40000.0)
    D = 16
    z = c[..., D - rope_dim::2] + 1j * c[..., D - rope_dim + 1::2]
    j = np.arange(11)[None, :, None]
    theta = 40000.0 ** (-np.arange(0, rope_dim, 2) / rope_dim)
    zr = z * np.exp(1j * j * theta)
    np.testing.assert_allclose(got[..., :D - rope_dim], c[..., :D - rope_dim], rtol=0, atol=0)
    np.testing.assert_allclose(got[..., D - rope_dim::2], zr.real, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got[..., D - rope_dim + 1::2], zr.imag, rtol=1e-12, atol=1e-13)


def test_rotation_depends_on_relative_position_only():
    # <R_m a, R_n b> = <R_(m-n) a, b> on the rotated channels
    a = rnd(8)
    b = rnd(8)
    rows = np.zeros((1, 20, 8))
    rows[0, :] = a
    ra = ep.epilogue(rows, None, 0.0, 8, 10.0)[0]
    rowsb = np.zeros((1, 20, 8))
    rowsb[0, :] = b
    rb = ep.epilogue(rowsb, None, 0.0, 8, 10.0)[0]
    for m, n in [(7, 3), (15, 11), (4, 0), (19, 15)]:
        assert np.dot(ra[m], rb[n]) == pytest.approx(np.dot(ra[m - n], b), rel=1e-11, abs=1e-12)


def test_identity_cases():
    c = rnd(1, 5, 8)
    np.testing.assert_array_equal(ep.epilogue(c, None, 1e-6, 0, 40000.0), c)
    # position 0 is not rotated
    out = ep.epilogue(c, None, 0.0, 8, 40000.0)
    np.testing.assert_allclose(out[0, 0], c[0, 0], rtol=0, atol=1e-15)
    # unit weight: rotation keeps the rms, the norm makes it sqrt(m / (m + eps))
    out = ep.epilogue(c, np.ones(8), 1e-3, 4, 40000.0)
    ms = np.mean(c * c, axis=-1)
    np.testing.assert_allclose(np.mean(out * out, axis=-1), ms / (ms + 1e-3), rtol=1e-12)


def _torch_pool(x, z, r, L):
    b, S, D = x.shape
    rows = []
    for j in range(S // r):
        lo, hi = max(0, (j + 1) * r - L), (j + 1) * r
        a = torch.softmax(z[:, lo:hi].expand(-1, -1, D), dim=1)
        rows.append((a * x[:, lo:hi]).sum(dim=1))
    return torch.stack(rows, dim=1)


def _torch_epilogue(c, w, eps, rope_dim, base):
    D = c.shape[-1]
    y = torch.nn.functional.rms_norm(c, (D,), w, eps=eps) if w is not None else c
    if rope_dim == 0:
        return y
    keep, rot = y[..., :D - rope_dim], y[..., D - rope_dim:]
    zc = torch.view_as_complex(rot.reshape(*rot.shape[:-1], rope_dim // 2, 2).contiguous())
    j = torch.arange(c.shape[1], dtype=torch.float64)[:, None]
    theta = base ** (-torch.arange(0, rope_dim, 2, dtype=torch.float64) / rope_dim)
    zr = zc * torch.polar(torch.ones_like(j * theta), j * theta)
    return torch.cat([keep, torch.view_as_real(zr).reshape(rot.shape)], dim=-1)


@pytest.mark.parametrize("zc,with_norm,rope_dim", [(16, True, 8), (1, True, 16), (16, False, 8), (1, True, 0)])
def test_backward_through_pooling_against_torch_autograd(zc, with_norm, rope_dim):
    r, L, S, D = 4, 8, 30, 16
    x, z, w = rnd(2, S, D), rnd(2, S, zc), rnd(D)
    dout = rnd(2, S // r, D)
    eps, base = 1e-5, 40000.0
    c32 = oracle.compress(x, z, r, L)
    out = ep.epilogue(c32, w if with_norm else None, eps, rope_dim, base)
    dc32, dw = ep.epilogue_bwd(c32, w if with_norm else None, eps, rope_dim, base, dout)
    dx, dz = oracle.compress_bwd(x, z, dc32, r, L)
    tx = torch.tensor(x, requires_grad=True)
    tz = torch.tensor(z, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    tout = _torch_epilogue(_torch_pool(tx, tz, r, L), tw if with_norm else None, eps, rope_dim, base)
    (tout * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(out, tout.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dz, tz.grad.numpy(), rtol=1e-10, atol=1e-12)
    if with_norm:
        np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-12)
    else:
        assert dw is None
