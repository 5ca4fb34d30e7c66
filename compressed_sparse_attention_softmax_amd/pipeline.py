"""One pass of the CSA hot path through the C ABI: allocation and call order only.

    compress -> index_topk -> sparse_attn_fwd -> sparse_attn_bwd -> compress_bwd

All calls go to the same HIP stream with no host synchronisation in between.
The compressed rows produced by ``csa_compress`` feed the attention, and the
compressed-row gradient of the attention backward feeds the compressor
backward.  With ``topk == 0`` the indexer is skipped and the attention runs in
dense mode over every valid compressed row (the heavy-compression layer).

``indexer_loss`` is the indexer's training path: after the attention forward
it consumes the selected blocks, their scores and the attention LSE and
produces the distillation loss per query row and its gradients into the
indexer's inputs.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _abi as abi


@dataclasses.dataclass
class Buffers:
    c: torch.Tensor
    c32: Optional[torch.Tensor]
    idx: Optional[torch.Tensor]
    score: Optional[torch.Tensor]
    out: torch.Tensor
    lse: torch.Tensor
    dq: torch.Tensor
    dkv: torch.Tensor
    dc: torch.Tensor
    dsink: Optional[torch.Tensor]
    dx: torch.Tensor
    dz: torch.Tensor
    ws: torch.Tensor        # attention-backward workspace (csa_sparse_attn_bwd_workspace bytes)


def allocate(dims: abi.csa_dims, dtype: torch.dtype, z_channels: int, device="cuda",
             with_sink: bool = True, with_c32: bool = False, with_score: bool = True) -> Buffers:
    b, S, H, D = dims.b, dims.sq, dims.h, dims.d
    nc = abi.n_compressed(dims)
    kp = abi.kprime(dims) if dims.topk > 0 else 0
    f32 = torch.float32
    e = dict(device=device)
    return Buffers(
        c=torch.empty(b, nc, D, dtype=dtype, **e),
        c32=torch.empty(b, nc, D, dtype=f32, **e) if with_c32 else None,
        idx=torch.empty(b, S, kp, dtype=torch.int32, **e) if kp > 0 else None,
        score=torch.empty(b, S, kp, dtype=f32, **e) if (kp > 0 and with_score) else None,
        out=torch.empty(b, S, H, D, dtype=dtype, **e),
        lse=torch.empty(b, S, H, dtype=f32, **e),
        dq=torch.empty(b, S, H, D, dtype=dtype, **e),
        dkv=torch.empty(b, S, D, dtype=f32, **e),
        dc=torch.empty(b, nc, D, dtype=f32, **e),
        dsink=torch.empty(H, dtype=f32, **e) if with_sink else None,
        dx=torch.empty(b, S, D, dtype=f32, **e),
        dz=torch.empty(b, S, z_channels, dtype=f32, **e),
        ws=torch.empty(max(abi.csa_sparse_attn_bwd_workspace(dims), 16), dtype=torch.uint8, **e),
    )


def forward(dims, inp, buf: Buffers, scale: float, stream=None) -> None:
    abi.csa_compress(dims, inp["x"], inp["z"], buf.c, buf.c32, stream=stream)
    if buf.idx is not None:
        abi.csa_index_topk(dims, inp["q_i"], inp["k_i"], inp["w"], buf.idx, buf.score, stream=stream)
    abi.csa_sparse_attn_fwd(dims, inp["q"], inp["kv"], buf.c, buf.idx, inp.get("sink"), scale,
                            buf.out, buf.lse, stream=stream)


def backward(dims, inp, buf: Buffers, scale: float, stream=None) -> None:
    abi.csa_sparse_attn_bwd(dims, inp["q"], inp["kv"], buf.c, buf.idx, inp.get("sink"), scale, buf.out,
                            buf.lse, inp["do"], buf.dq, buf.dkv, buf.dc,
                            buf.dsink if inp.get("sink") is not None else None, ws=buf.ws, stream=stream)
    abi.csa_compress_bwd(dims, inp["x"], inp["z"], buf.dc, buf.dx, buf.dz, stream=stream)


def step(dims, inp, buf: Buffers, scale: float, stream=None) -> None:
    forward(dims, inp, buf, scale, stream)
    backward(dims, inp, buf, scale, stream)


@dataclasses.dataclass
class LossBuffers:
    kl: torch.Tensor
    dq_i: torch.Tensor
    dw: torch.Tensor
    dk_i: torch.Tensor
    ws: torch.Tensor        # csa_indexer_loss_workspace bytes


def allocate_loss(dims: abi.csa_dims, dtype: torch.dtype, device="cuda") -> LossBuffers:
    b, S = dims.b, dims.sq
    nc = abi.n_compressed(dims)
    f32 = torch.float32
    e = dict(device=device)
    return LossBuffers(
        kl=torch.empty(b, S, dtype=f32, **e),
        dq_i=torch.empty(b, S, dims.idx_heads, dims.idx_dim, dtype=dtype, **e),
        dw=torch.empty(b, S, dims.idx_heads, dtype=f32, **e),
        dk_i=torch.empty(b, nc, dims.idx_dim, dtype=f32, **e),
        ws=torch.empty(max(abi.csa_indexer_loss_workspace(dims), 16), dtype=torch.uint8, **e),
    )


def indexer_loss(dims, inp, buf: Buffers, lbuf: LossBuffers, scale: float, dkl, c=None, stream=None) -> None:
    """Distillation loss of the indexer over the blocks ``buf.idx`` selected, with
    the attention LSE ``buf.lse``; ``dkl`` [b, sq] weights each row's loss."""
    abi.csa_indexer_loss(dims, inp["q"], buf.c if c is None else c, buf.lse, inp["q_i"], inp["k_i"], inp["w"],
                         buf.idx, buf.score, scale, kl=lbuf.kl, dkl=dkl, dq_i=lbuf.dq_i, dw=lbuf.dw,
                         dk_i=lbuf.dk_i, ws=lbuf.ws, stream=stream)
