"""Seeded synthetic inputs for the compressed-sparse-attention hot path.

This module only draws random tensors: it holds none of the method's
arithmetic and is shared by the tests, the benchmark and the oracle checks,
so both sides of every comparison see the very same input values.

Each tensor comes from its own ``torch.Generator`` seeded with
``seed * 1000 + tensor_id``.  Values are drawn as float32 standard normals,
scaled, and then rounded once to the working dtype (round-to-nearest-even).
Drawing on ``device="cuda"`` keeps large configurations resident in HBM; the
oracle side receives ``.cpu()`` copies of exactly those values.

The five workloads follow the shapes of the pages' CSA layers (DeepSeek-V4
style compressed sparse attention: one shared KV head, a sliding window, a
ratio-r compressor, a learned indexer with top-k and a per-head sink).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

# tensor ids; the order is part of the recipe
_T_Q, _T_KV, _T_X, _T_Z, _T_QI, _T_KI, _T_W, _T_SINK, _T_DO, _T_SKEW = range(10)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    b: int
    sq: int
    h: int
    d: int
    ratio: int
    span: int
    window: int
    idx_heads: int
    idx_dim: int
    topk: int           # 0 => no indexer: attend densely over valid compressed rows
    dtype: str          # "f32" or "bf16"
    z_channels: int     # 1 (one pooling score per row) or d (one per channel)
    # value scales (standard deviations) of the drawn tensors
    s_q: float = 1.0
    s_kv: float = 1.0
    s_x: float = 1.0
    s_z: float = 1.0
    s_qi: float = 1.0
    s_ki: float = 1.0
    s_w: float = 1.0
    s_sink: float = 1.0
    s_do: float = 1.0
    skew_frac: float = 0.0   # fraction of indexer keys per batch that are scaled
    skew_mult: float = 1.0

    @property
    def n_c(self) -> int:
        return self.sq // self.ratio

    @property
    def kprime(self) -> int:
        return min(self.topk, self.n_c) if self.topk > 0 else 0

    @property
    def scale(self) -> float:
        return self.d ** -0.5

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 CSA layer
    "tiny_f32": Workload("tiny_f32", b=1, sq=256, h=4, d=64, ratio=4, span=4, window=16,
                         idx_heads=2, idx_dim=32, topk=16, dtype="f32", z_channels=64),
    # CSA-4 layer, overlapping pooling (stride 4, span 8)
    "csa4_s4096": Workload("csa4_s4096", b=1, sq=4096, h=64, d=128, ratio=4, span=8, window=128,
                           idx_heads=64, idx_dim=128, topk=512, dtype="bf16", z_channels=128,
                           s_q=0.5, s_kv=0.5, s_x=0.5, s_qi=0.5, s_ki=0.5, s_w=0.125),
    # CSA-4 at head_dim 512
    "csa4_d512_s8192": Workload("csa4_d512_s8192", b=1, sq=8192, h=64, d=512, ratio=4, span=4,
                                window=128, idx_heads=64, idx_dim=128, topk=1024, dtype="bf16",
                                z_channels=512, s_w=0.125),
    # HCA-128: heavy compression, no indexer
    "hca128_s16384": Workload("hca128_s16384", b=1, sq=16384, h=64, d=512, ratio=128, span=128,
                              window=128, idx_heads=64, idx_dim=128, topk=0, dtype="bf16",
                              z_channels=512, s_z=0.1, s_w=0.125),
    # long context, skewed indexer keys (scatter stress)
    "csa4_s65536_skew": Workload("csa4_s65536_skew", b=2, sq=65536, h=64, d=128, ratio=4, span=4,
                                 window=128, idx_heads=64, idx_dim=128, topk=2048, dtype="bf16",
                                 z_channels=128, s_w=0.125, skew_frac=0.1, skew_mult=4.0),
}

# order of the five workloads as listed for the method
WORKLOAD_ORDER = ["tiny_f32", "csa4_s4096", "csa4_d512_s8192", "hca128_s16384", "csa4_s65536_skew"]
WORKLOAD_SEEDS = {name: i + 1 for i, name in enumerate(WORKLOAD_ORDER)}


def _gen(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + tid)
    return g


def _normal(shape, std, seed, tid, device, dtype):
    g = _gen(seed, tid, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def skewed_blocks(wl: Workload, seed: int, device="cpu") -> torch.Tensor:
    """Per batch, the sorted indices of the indexer keys that are scaled."""
    n = int(wl.skew_frac * wl.n_c)
    g = _gen(seed, _T_SKEW, "cpu")
    rows = [torch.randperm(wl.n_c, generator=g)[:n].sort().values for _ in range(wl.b)]
    return torch.stack(rows).to(device) if n > 0 else torch.zeros(wl.b, 0, dtype=torch.int64, device=device)


def make_inputs(wl: Workload, seed: int, device="cpu", parts=("attn", "compress", "index", "bwd"),
                with_sink: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Draw the inputs of one workload.

    Returns a dict with (some of) ``q [b,sq,h,d]``, ``kv [b,sq,d]``,
    ``x [b,sq,d]``, ``z [b,sq,z_channels]``, ``q_i [b,sq,idx_heads,idx_dim]``,
    ``k_i [b,n_c,idx_dim]``, ``w [b,sq,idx_heads]`` (float32),
    ``sink [h]`` (float32) and ``do [b,sq,h,d]``.
    """
    dt = wl.torch_dtype
    out: Dict[str, Optional[torch.Tensor]] = {}
    if "attn" in parts:
        out["q"] = _normal((wl.b, wl.sq, wl.h, wl.d), wl.s_q, seed, _T_Q, device, dt)
        out["kv"] = _normal((wl.b, wl.sq, wl.d), wl.s_kv, seed, _T_KV, device, dt)
        out["sink"] = (_normal((wl.h,), wl.s_sink, seed, _T_SINK, device, torch.float32)
                       if with_sink else None)
    if "compress" in parts:
        out["x"] = _normal((wl.b, wl.sq, wl.d), wl.s_x, seed, _T_X, device, dt)
        out["z"] = _normal((wl.b, wl.sq, wl.z_channels), wl.s_z, seed, _T_Z, device, dt)
    if "index" in parts and wl.topk > 0:
        out["q_i"] = _normal((wl.b, wl.sq, wl.idx_heads, wl.idx_dim), wl.s_qi, seed, _T_QI, device, dt)
        ki = _normal((wl.b, wl.n_c, wl.idx_dim), wl.s_ki, seed, _T_KI, device, torch.float32)
        if wl.skew_frac > 0:
            blocks = skewed_blocks(wl, seed, device)
            for bi in range(wl.b):
                ki[bi, blocks[bi]] *= wl.skew_mult
        out["k_i"] = ki.to(dt)
        out["w"] = _normal((wl.b, wl.sq, wl.idx_heads), wl.s_w, seed, _T_W, device, torch.float32)
    if "bwd" in parts:
        out["do"] = _normal((wl.b, wl.sq, wl.h, wl.d), wl.s_do, seed, _T_DO, device, dt)
    return out


def random_topk_indices(wl: Workload, seed: int, device="cpu", repeat_frac: float = 0.0) -> torch.Tensor:
    """A structurally valid index list ``[b,sq,K']`` drawn at random.

    Row t holds ``min(K', n_valid(t))`` distinct valid blocks in ascending
    order followed by -1 padding.  Used to drive the attention stage on its own.
    Only random draws happen here; the validity bound ``(t+1)//ratio`` is part
    of the input contract, stated in the C header.
    """
    kp = wl.kprime
    g = _gen(seed, 50, "cpu")
    idx = torch.full((wl.b, wl.sq, kp), -1, dtype=torch.int32)
    keys = torch.rand((wl.b, wl.sq, wl.n_c), generator=g)
    for bi in range(wl.b):
        for t in range(wl.sq):
            nv = (t + 1) // wl.ratio
            m = min(kp, nv)
            if m == 0:
                continue
            sel = torch.topk(keys[bi, t, :nv], m).indices.sort().values
            idx[bi, t, :m] = sel.to(torch.int32)
    return idx.to(device)


def packed_doc_ids(b: int, sq: int, mean_len: float, seed: int, device="cpu") -> torch.Tensor:
    """Document ids ``[b,sq]`` int32 for sequences packed from several documents.

    Document lengths are drawn from an exponential length mix with the given
    mean (at least one token each), so segment starts fall anywhere, not only
    on compression-block boundaries.  Ids increase along a row and differ
    between batch rows.  Only random draws happen here.
    """
    g = _gen(seed, 60, "cpu")
    doc = torch.empty(b, sq, dtype=torch.int32)
    for bi in range(b):
        pos, k = 0, 0
        while pos < sq:
            n = max(1, int(torch.empty(1).exponential_(1.0 / mean_len, generator=g).item()))
            doc[bi, pos:pos + n] = 1000 * bi + k
            pos += n
            k += 1
    return doc.to(device)


@dataclasses.dataclass(frozen=True)
class GqaWorkload:
    """Shapes of the simplified DSA over grouped-query attention: a one-head
    indexer at full resolution selects ``topk`` keys per query; attention
    over those keys with ``h`` query heads sharing ``h_kv`` key/value heads."""
    name: str
    b: int
    sq: int
    h: int
    h_kv: int
    d_qk: int
    d_v: int
    topk: int
    idx_dim: int
    dtype: str

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def kprime(self) -> int:
        return min(self.topk, self.sq)

    @property
    def scale(self) -> float:
        return self.d_qk ** -0.5

    def replace(self, **kw) -> "GqaWorkload":
        return dataclasses.replace(self, **kw)


GQA_WORKLOADS = {
    "dsa_gqa_tiny_f32": GqaWorkload("dsa_gqa_tiny_f32", 2, 200, 8, 2, 32, 32, 24, 32, "f32"),
    "dsa_gqa_s4096": GqaWorkload("dsa_gqa_s4096", 1, 4096, 32, 8, 128, 128, 512, 128, "bf16"),
}


def make_gqa_inputs(wl: GqaWorkload, seed: int, device="cpu") -> Dict[str, torch.Tensor]:
    """q [b,sq,h,d_qk], k [b,sq,h_kv,d_qk], v [b,sq,h_kv,d_v], dO [b,sq,h,d_v],
    and the one-head indexer's q_i [b,sq,1,idx_dim], k_i [b,sq,idx_dim]:
    standard normals (q_i, k_i scaled by 0.5), rounded once to the dtype."""
    dt = wl.torch_dtype
    b, S = wl.b, wl.sq
    return {
        "q": _normal((b, S, wl.h, wl.d_qk), 1.0, seed, 70, device, dt),
        "k": _normal((b, S, wl.h_kv, wl.d_qk), 1.0, seed, 71, device, dt),
        "v": _normal((b, S, wl.h_kv, wl.d_v), 1.0, seed, 72, device, dt),
        "do": _normal((b, S, wl.h, wl.d_v), 1.0, seed, 73, device, dt),
        "q_i": _normal((b, S, 1, wl.idx_dim), 0.5, seed, 74, device, dt),
        "k_i": _normal((b, S, wl.idx_dim), 0.5, seed, 75, device, dt),
    }
