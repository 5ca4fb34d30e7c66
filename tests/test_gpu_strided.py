"""Strided attention calls: sequence-major (SBHD) and head-padded views give
the same results, bit for bit, as the contiguous calls on the same values,
and (on a small fp32 case) agree with the oracle.

Every call goes through the C ABI (``libcsa.so``); inputs come from
``csa_synth``.
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


def _view(t, layout, pad=0):
    """A view of t ([b, s, ...]) with the same values in another layout:
    'sbhd' (sequence-major storage) or 'pad' (last axis padded by `pad`)."""
    if layout == "sbhd":
        store = torch.empty((t.shape[1], t.shape[0]) + tuple(t.shape[2:]), dtype=t.dtype, device=t.device)
        v = store.transpose(0, 1)
    else:
        store = torch.full(tuple(t.shape[:-1]) + (t.shape[-1] + pad,), float("nan"), dtype=t.dtype, device=t.device)
        v = store[..., :t.shape[-1]]
    v.copy_(t)
    return v


def _empty_like_layout(shape, dtype, layout, pad=0, fill=3.0):
    b, s = shape[0], shape[1]
    if layout == "sbhd":
        return torch.full((s, b) + tuple(shape[2:]), fill, dtype=dtype, device="cuda").transpose(0, 1)
    store = torch.full(tuple(shape[:-1]) + (shape[-1] + pad,), fill, dtype=dtype, device="cuda")
    return store[..., :shape[-1]]


def _run(csa, dm, wl, q, kv, c, idx, sink, do, layout=None, pad=0):
    b, S, H, D = wl.b, wl.sq, wl.h, wl.d
    strided = layout is not None
    mk = (lambda shape, dt: _empty_like_layout(shape, dt, layout, pad)) if strided else \
        (lambda shape, dt: torch.full(shape, 3.0, dtype=dt, device="cuda"))
    if strided:
        q, do = _view(q, layout, pad), _view(do, layout, pad)
        kv = _view(kv, layout, pad)
    out = mk((b, S, H, D), q.dtype)
    lse = (_empty_like_layout((b, S, H), torch.float32, layout, 4) if strided
           else torch.empty(b, S, H, device="cuda"))
    dq = mk((b, S, H, D), q.dtype)
    dkv = mk((b, S, D), torch.float32)
    dc = torch.full((b, wl.n_c, D), 3.0, device="cuda") if c is not None else None
    dsink = torch.full((H,), 3.0, device="cuda") if sink is not None else None
    ws = torch.empty(csa.csa_sparse_attn_bwd_workspace(dm), dtype=torch.uint8, device="cuda")
    if strided:
        csa.csa_sparse_attn_fwd_strided(dm, q, kv, c, idx, sink, wl.scale, out, lse)
        csa.csa_sparse_attn_bwd_strided(dm, q, kv, c, idx, sink, wl.scale, out, lse, do, dq, dkv, dc, dsink, ws=ws)
    else:
        csa.csa_sparse_attn_fwd(dm, q, kv, c, idx, sink, wl.scale, out, lse)
        csa.csa_sparse_attn_bwd(dm, q, kv, c, idx, sink, wl.scale, out, lse, do, dq, dkv, dc, dsink, ws=ws)
    torch.cuda.synchronize()
    return dict(out=out.contiguous(), lse=lse.contiguous(), dq=dq.contiguous(), dkv=dkv.contiguous(), dc=dc,
                dsink=dsink)


STRIDED_CASES = [
    ("tiny_f32_sbhd", TINY.replace(b=2), "sbhd", 0, "random"),
    ("csa4_bf16_b2_h48_sbhd", CSA4_SMALL.replace(b=2, sq=333, h=48, topk=40), "sbhd", 0, "random"),
    ("csa4_bf16_b3_h8_sbhd", CSA4_SMALL.replace(b=3, sq=290, h=8, topk=40), "sbhd", 0, "random"),
    ("csa4_bf16_b2_pad", CSA4_SMALL.replace(b=2, sq=260, h=17, topk=40), "pad", 16, "random"),
    ("csa4_bf16_b2_dense_sbhd", CSA4_SMALL.replace(b=2, sq=300), "sbhd", 0, "dense"),
    ("csa4_bf16_b2_window_only_sbhd", CSA4_SMALL.replace(b=2, sq=300), "sbhd", 0, "window"),
    ("d512_bf16_b2_sbhd", D512_SMALL.replace(b=2, sq=200), "sbhd", 0, "random"),
    ("bf16_d64_b2_sbhd", CSA4_SMALL.replace(b=2, sq=300, h=16, d=64, z_channels=64, topk=40), "sbhd", 0, "random"),
]


@pytest.mark.parametrize("name,wl,layout,pad,mode", STRIDED_CASES, ids=[c[0] for c in STRIDED_CASES])
def test_strided_attention_matches_contiguous(gpu, name, wl, layout, pad, mode):
    import compressed_sparse_attention_softmax_amd as csa
    say(f"[strided] {name} b={wl.b} sq={wl.sq} h={wl.h} d={wl.d} layout={layout} pad={pad} mode={mode}")
    inp = csa_synth.make_inputs(wl, 23, device="cuda", parts=("attn", "bwd"))
    g = torch.Generator().manual_seed(29)
    c = None
    if mode != "window":
        c = (torch.randn(wl.b, wl.n_c, wl.d, generator=g) * 0.5).to(wl.torch_dtype).cuda()
    idx = csa_synth.random_topk_indices(wl, 24).cuda() if mode == "random" else None
    dm = csa.dims_of(wl)
    ref = _run(csa, dm, wl, inp["q"], inp["kv"], c, idx, inp["sink"], inp["do"])
    got = _run(csa, dm, wl, inp["q"], inp["kv"], c, idx, inp["sink"], inp["do"], layout=layout, pad=pad)
    for k in ("out", "lse", "dq", "dkv", "dc", "dsink"):
        if ref[k] is None:
            continue
        assert torch.equal(got[k], ref[k]), f"{k}: strided call differs from the contiguous call"
    if name == "tiny_f32_sbhd":
        b, S, H, D = wl.b, wl.sq, wl.h, wl.d
        rows = oracle.all_rows(b, S)
        q64 = f64(inp["q"]).reshape(b * S, H, D)
        ii = idx.cpu().numpy().reshape(b * S, -1)
        sink = f64(inp["sink"])
        ro, rl = oracle.attn_fwd(q64, f64(inp["kv"]), f64(c), ii, sink, wl.scale, wl.window, wl.ratio, rows)
        rdq, rdkv, rdc, rds = oracle.attn_bwd(q64, f64(inp["kv"]), f64(c), ii, sink, wl.scale, wl.window,
                                              wl.ratio, rows, f64(inp["do"]).reshape(b * S, H, D))
        tol = tol_of(wl.torch_dtype)
        check_close("out", got["out"].reshape(b * S, H, D), ro, tol)
        check_close("lse", got["lse"].reshape(b * S, H), rl, tol)
        check_close("dq", got["dq"].reshape(b * S, H, D), rdq, tol)
        check_close("dkv", got["dkv"], rdkv, tol)
        check_close("dc", got["dc"], rdc, tol)
        check_close("dsink", got["dsink"], rds, tol)


def test_strided_binding_rejects_mismatched_output_strides(gpu):
    import compressed_sparse_attention_softmax_amd as csa
    wl = TINY.replace(b=2)
    inp = csa_synth.make_inputs(wl, 5, device="cuda", parts=("attn",))
    dm = csa.dims_of(wl)
    q = _view(inp["q"], "sbhd")
    kv = _view(inp["kv"], "sbhd")
    out = torch.empty(wl.b, wl.sq, wl.h, wl.d, device="cuda")       # contiguous, q is not
    lse = torch.empty(wl.b, wl.sq, wl.h, device="cuda")
    with pytest.raises(ValueError, match="differ"):
        csa.csa_sparse_attn_fwd_strided(dm, q, kv, None, None, inp["sink"], wl.scale, out, lse)
