"""The backward's key-stationary pass keeps every query's contribution.

The dK/dV (dC) kernel walks each block of consecutive queries over a tile of
key rows and accumulates in registers; the first and the last query of a
block are where a lost or doubled contribution would hide (the loop's entry
and exit).  Here dO is zero except on the first (or the last) query of every
block, so dkv and dc consist of those queries' contributions alone and any
one of them missing fails the bar by far.  Shapes: d = 512 (two staged head
units per query), d = 128 with selected rows, dense mode and window only.
"""
import numpy as np
import pytest
import torch

import csa_synth
import oracle
from parity import check_close, f64, say, tol_of

pytestmark = pytest.mark.gpu

W = csa_synth.WORKLOADS
CSA4_SMALL = W["csa4_s4096"].replace(sq=1030, topk=96)
D512_SMALL = W["csa4_d512_s8192"].replace(sq=300, topk=40)


def _edge_case(wl, which, mode, seed=71):
    import compressed_sparse_attention_softmax_amd as csa
    inp = csa_synth.make_inputs(wl, seed, device="cuda", parts=("attn", "compress", "bwd"))
    b, S, H, D, nc = wl.b, wl.sq, wl.h, wl.d, wl.n_c
    dm = csa.dims_of(wl)
    c = None
    if mode != "window":
        c = torch.tensor(oracle.compress(f64(inp["x"]), f64(inp["z"]), wl.ratio, wl.span)).to(wl.torch_dtype).cuda()
    idx = csa_synth.random_topk_indices(wl, seed + 1).cuda() if mode == "selected" else None
    qb = csa.csa_sparse_attn_bwd_query_block(dm, c is not None)
    assert qb > 0
    t = np.arange(S)
    keep = (t % qb == 0) if which == "first" else ((t % qb == qb - 1) | (t == S - 1))
    say(f"  query block {qb}: dO kept on {int(keep.sum())} of {S} queries ({which} of each block)")
    do = inp["do"].clone()
    do[:, torch.as_tensor(~keep, device="cuda")] = 0
    out = torch.empty(b, S, H, D, dtype=wl.torch_dtype, device="cuda")
    lse = torch.empty(b, S, H, device="cuda")
    csa.csa_sparse_attn_fwd(dm, inp["q"], inp["kv"], c, idx, inp["sink"], wl.scale, out, lse)
    dq = torch.empty_like(out)
    dkv = torch.full((b, S, D), 3.0, device="cuda")
    dc = torch.full((b, nc, D), 3.0, device="cuda") if c is not None else None
    dsink = torch.full((H,), 3.0, device="cuda")
    ws = torch.empty(csa.csa_sparse_attn_bwd_workspace(dm), dtype=torch.uint8, device="cuda")
    csa.csa_sparse_attn_bwd(dm, inp["q"], inp["kv"], c, idx, inp["sink"], wl.scale, out, lse, do, dq, dkv, dc,
                            dsink, ws=ws)
    torch.cuda.synchronize()
    rows = oracle.all_rows(b, S)
    q64 = f64(inp["q"]).reshape(b * S, H, D)
    cc = f64(c) if c is not None else np.zeros((b, 0, D))
    ii = None if idx is None else idx.cpu().numpy().reshape(b * S, -1)
    rdq, rdkv, rdc, rds = oracle.attn_bwd(q64, f64(inp["kv"]), cc, ii, f64(inp["sink"]), wl.scale, wl.window,
                                          wl.ratio, rows, f64(do).reshape(b * S, H, D))
    tol = tol_of(wl.torch_dtype)
    check_close("dq", dq.reshape(b * S, H, D), rdq, tol)
    check_close("dkv", dkv, rdkv, tol)
    if dc is not None:
        check_close("dc", dc, rdc, tol)
    check_close("dsink", dsink, rds, tol)
    # rows no kept query reaches are exactly zero
    assert torch.all(dkv.cpu()[torch.as_tensor(np.abs(rdkv) == 0)] == 0)


EDGE_CASES = [
    ("d512_selected", D512_SMALL, "selected"),
    ("d512_dense", D512_SMALL.replace(sq=260), "dense"),
    ("d128_selected", CSA4_SMALL.replace(sq=700), "selected"),
    ("d128_dense", CSA4_SMALL.replace(sq=600), "dense"),
    ("d128_window_only", CSA4_SMALL.replace(sq=500), "window"),
]


@pytest.mark.parametrize("which", ["first", "last"])
@pytest.mark.parametrize("name,wl,mode", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_every_block_edge_query_contributes(gpu, name, wl, mode, which):
    say(f"[block edges] {name} sq={wl.sq} d={wl.d} mode={mode} {which}")
    _edge_case(wl, which, mode)
