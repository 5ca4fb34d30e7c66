"""GPU parity of the dense warm-up form of the indexer loss
(``csa_indexer_loss_dense``) against the fp64 oracle
(``oracle.indexer_loss.dense_warmup_loss``), through the C ABI.

Each case runs twice: on the smallest workspace the plan accepts (the
queries in many chunks) and on one that holds every query at once.  Both
are checked against the oracle; kl, dq_i and dw do not depend on the
chunking (bit-identical), dk_i sums the chunks in another order.
"""
import numpy as np
import pytest
import torch

import csa_synth
import oracle
from parity import check_close, f64, say, tol_of

pytestmark = pytest.mark.gpu

W = csa_synth.WORKLOADS
TINY = W["tiny_f32"]
CSA4_SMALL = W["csa4_s4096"].replace(sq=1030, topk=96)
D512_SMALL = W["csa4_d512_s8192"].replace(sq=300, topk=40)


def _run(csa, dm, wl, cu, inp, c, lse, dkl, grads, ws_bytes):
    b, S, nc = wl.b, wl.sq, wl.n_c
    kl = torch.full((b, S), 7.0, device="cuda")
    out = {}
    if grads:
        out = dict(dq_i=torch.full((b, S, wl.idx_heads, wl.idx_dim), 7.0, dtype=wl.torch_dtype, device="cuda"),
                   dw=torch.full((b, S, wl.idx_heads), 7.0, device="cuda"),
                   dk_i=torch.full((b, nc, wl.idx_dim), 7.0, device="cuda"))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    csa.csa_indexer_loss_dense(dm, cu(inp["q"]), cu(c), cu(lse), cu(inp["q_i"]), cu(inp["k_i"]), cu(inp["w"]),
                               wl.scale, kl=kl, dkl=cu(dkl) if grads else None, ws=ws, **out)
    torch.cuda.synchronize()
    out["kl"] = kl
    return out


def _dense_case(wl, seed, grads=True):
    import compressed_sparse_attention_softmax_amd as csa
    from oracle import indexer_loss as il
    inp = csa_synth.make_inputs(wl, seed, device="cpu", parts=("attn", "compress", "index"))
    b, S, H, D, nc = wl.b, wl.sq, wl.h, wl.d, wl.n_c
    dt = wl.torch_dtype
    c = torch.tensor(oracle.compress(f64(inp["x"]), f64(inp["z"]), wl.ratio, wl.span)).to(dt)
    rows = oracle.all_rows(b, S)
    q64 = f64(inp["q"]).reshape(b * S, H, D)
    # the warm-up's attention attends every valid block: its LSE, rounded once
    _, lse64 = oracle.attn_fwd(q64, f64(inp["kv"]), f64(c), None, f64(inp["sink"]), wl.scale, wl.window,
                               wl.ratio, rows)
    lse = torch.tensor(lse64, dtype=torch.float32).reshape(b, S, H)
    dkl = torch.randn(b, S, generator=torch.Generator().manual_seed(seed + 5))
    dm = csa.dims_of(wl)
    cu = lambda a: torch.as_tensor(a).cuda()
    least = csa.csa_indexer_loss_dense_workspace(dm, 0)
    full = csa.csa_indexer_loss_dense_workspace(dm, 1 << 40)
    say(f"  workspace: least {least} B, all queries {full} B")
    small = _run(csa, dm, wl, cu, inp, c, lse, dkl, grads, least)
    big = _run(csa, dm, wl, cu, inp, c, lse, dkl, grads, full)
    ref = il.dense_warmup_loss(q64, f64(c), f64(lse).reshape(b * S, H), f64(inp["q_i"]).reshape(b * S, wl.idx_heads,
                               wl.idx_dim), f64(inp["k_i"]), f64(inp["w"]).reshape(b * S, wl.idx_heads), wl.scale,
                               wl.ratio, rows, dkl=dkl.double().numpy().reshape(-1) if grads else None)
    tol = tol_of(dt)
    for got in (small, big):
        check_close("kl", got["kl"].reshape(-1), ref["kl"], tol)
        if grads:
            check_close("dq_i", got["dq_i"].reshape(b * S, wl.idx_heads, wl.idx_dim), ref["dq_i"], tol)
            check_close("dw", got["dw"].reshape(b * S, wl.idx_heads), ref["dw"], tol)
            check_close("dk_i", got["dk_i"], ref["dk_i"], tol)
    for k in ("kl", "dq_i", "dw"):
        if k in small:
            assert torch.equal(small[k], big[k]), f"{k} depends on the chunking"


DENSE_CASES = [
    ("tiny_f32", TINY, {}),
    ("tiny_f32_kl_only", TINY.replace(b=2, sq=203), dict(grads=False)),
    ("csa4_bf16", CSA4_SMALL, {}),
    ("csa4_bf16_b2_h48", CSA4_SMALL.replace(b=2, sq=333, h=48), {}),
    ("idx_dim64_heads40", CSA4_SMALL.replace(idx_heads=40, idx_dim=64, sq=900), {}),
    ("d512_bf16", D512_SMALL, {}),
    ("shorter_than_ratio", TINY.replace(sq=3), {}),
    # more blocks than the selected form's 2048-entry limit
    ("bf16_nc2112", CSA4_SMALL.replace(sq=8448, h=8, d=64, z_channels=64, idx_heads=8, idx_dim=32), {}),
]


@pytest.mark.parametrize("name,wl,kw", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_indexer_loss_dense_warmup(gpu, name, wl, kw):
    say(f"[indexer_loss_dense] {name} b={wl.b} sq={wl.sq} n_c={wl.n_c} h={wl.h} d={wl.d} "
        f"h_i={wl.idx_heads} d_i={wl.idx_dim} {kw}")
    _dense_case(wl, 61, **kw)
