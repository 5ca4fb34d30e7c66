"""fp64 oracle of the compressor's epilogue: post-pool norm, then RoPE on the
compressed positions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Megatron-LM PR #6400: the pooled row is cast once to the working dtype and
normalised (the compressor's ``norm``, review thread on the pooling
weights); the compressed rows get a rotary embedding with its own base
(40000 in the layer configuration thread).  Readings taken where the pages
are silent: the norm is an RMS norm with a learned per-channel weight,
n = y / sqrt(mean(y^2) + eps) * weight; the rotary embedding turns the last
``rope_dim`` channels of block j's row in interleaved pairs (2i, 2i+1) by the
angle j * base^(-2i / rope_dim) (block j sits at compressed position j); the
norm comes first.  ``weight = None`` skips the norm, ``rope_dim = 0`` the
rotation.  The one cast to the working dtype is taken as the identity here.

Plain NumPy over whole arrays; library exp, sqrt, sin, cos only.
"""
from __future__ import annotations

import numpy as np


def _angles(nc, rope_dim, base):
    i = np.arange(rope_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / rope_dim)
    return np.arange(nc, dtype=np.float64)[:, None] * theta[None, :]      # [nc, rope_dim/2]


def _rotate(v, rope_dim, base, sign):
    """Rotate the last rope_dim channels of v [b, nc, D] by sign * angle."""
    if rope_dim == 0:
        return v.copy()
    out = v.copy()
    D = v.shape[-1]
    ang = sign * _angles(v.shape[1], rope_dim, base)[None]
    cos, sin = np.cos(ang), np.sin(ang)
    x0 = v[..., D - rope_dim::2]
    x1 = v[..., D - rope_dim + 1::2]
    out[..., D - rope_dim::2] = x0 * cos - x1 * sin
    out[..., D - rope_dim + 1::2] = x0 * sin + x1 * cos
    return out


def epilogue(c, weight, eps, rope_dim, base):
    """c [b, nc, D] pooled rows -> normalised and rotated rows."""
    y = np.asarray(c, np.float64)
    if weight is not None:
        w = np.asarray(weight, np.float64)
        y = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps) * w
    return _rotate(y, rope_dim, base, 1.0)


def epilogue_bwd(c, weight, eps, rope_dim, base, dout):
    """Gradient of sum(dout * epilogue(c)) -> (dc [b, nc, D], dweight [D] or None)."""
    y = np.asarray(c, np.float64)
    dn = _rotate(np.asarray(dout, np.float64), rope_dim, base, -1.0)       # transpose of a rotation
    if weight is None:
        return dn, None
    w = np.asarray(weight, np.float64)
    D = y.shape[-1]
    inv = 1.0 / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    dweight = np.sum(dn * y * inv, axis=(0, 1))
    g = dn * w
    dy = inv * g - inv ** 3 * y * np.sum(g * y, axis=-1, keepdims=True) / D
    return dy, dweight
