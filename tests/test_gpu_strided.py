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


def _run(csa, dm, wl, q, kv, c, idx, sink, do, layout=None, pad=0, doc=None):
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
        csa.csa_sparse_attn_fwd_strided(dm, q, kv, c, idx, sink, wl.scale, out, lse, doc_ids=doc)
        csa.csa_sparse_attn_bwd_strided(dm, q, kv, c, idx, sink, wl.scale, out, lse, do, dq, dkv, dc, dsink, ws=ws,
                                        doc_ids=doc)
    else:
        csa.csa_sparse_attn_fwd(dm, q, kv, c, idx, sink, wl.scale, out, lse, doc_ids=doc)
        csa.csa_sparse_attn_bwd(dm, q, kv, c, idx, sink, wl.scale, out, lse, do, dq, dkv, dc, dsink, ws=ws,
                                doc_ids=doc)
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
    ("csa4_bf16_b2_docs_sbhd", CSA4_SMALL.replace(b=2, sq=400, topk=40), "sbhd", 0, "docs"),
    ("csa4_bf16_b2_dense_docs_pad", CSA4_SMALL.replace(b=2, sq=333), "pad", 16, "dense_docs"),
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
    idx = csa_synth.random_topk_indices(wl, 24).cuda() if mode in ("random", "docs") else None
    doc = csa_synth.packed_doc_ids(wl.b, wl.sq, 90.0, 25).cuda() if mode in ("docs", "dense_docs") else None
    dm = csa.dims_of(wl)
    ref = _run(csa, dm, wl, inp["q"], inp["kv"], c, idx, inp["sink"], inp["do"], doc=doc)
    got = _run(csa, dm, wl, inp["q"], inp["kv"], c, idx, inp["sink"], inp["do"], layout=layout, pad=pad, doc=doc)
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


COMPRESS_CASES = [
    ("tiny_f32_sbhd", TINY.replace(b=2), "sbhd", 0, False),
    ("csa4_bf16_b3_sbhd", CSA4_SMALL.replace(b=3, sq=1030), "sbhd", 0, False),
    ("csa4_bf16_b2_pad_epilogue", CSA4_SMALL.replace(b=2, sq=517), "pad", 8, True),
    ("csa4_bf16_b2_gate1_sbhd", CSA4_SMALL.replace(b=2, sq=301, z_channels=1), "sbhd", 0, False),
    ("d512_bf16_b2_sbhd_epilogue", D512_SMALL.replace(b=2, sq=260), "sbhd", 0, True),
]


@pytest.mark.parametrize("name,wl,layout,pad,epi", COMPRESS_CASES, ids=[c[0] for c in COMPRESS_CASES])
def test_strided_compressor_matches_contiguous(gpu, name, wl, layout, pad, epi):
    """Sequence-major or padded x, z, dx and dz through the strided compressor
    calls: c, c32, dx, dz and dnorm_w equal the contiguous calls' bit for bit
    (rows past n_c * ratio included, which receive zero)."""
    import compressed_sparse_attention_softmax_amd as csa
    say(f"[strided compressor] {name} b={wl.b} sq={wl.sq} d={wl.d} zc={wl.z_channels} layout={layout} epi={epi}")
    inp = csa_synth.make_inputs(wl, 31, device="cuda", parts=("compress",))
    dm = csa.dims_of(wl)
    b, S, D, zc, nc = wl.b, wl.sq, wl.d, wl.z_channels, wl.n_c
    g = torch.Generator().manual_seed(37)
    dc = (torch.randn(b, nc, D, generator=g) * 0.5).cuda()
    ep = {}
    if epi:
        ep = dict(norm_w=(1.0 + 0.1 * torch.randn(D, generator=g)).cuda(), rope_dim=min(64, D))
    ws = torch.empty(max(csa.csa_compress_bwd_workspace(dm), 16), dtype=torch.uint8, device="cuda")

    def run(strided):
        x, z = inp["x"], inp["z"]
        mk = (lambda shape: _empty_like_layout(shape, torch.float32, layout, pad)) if strided else \
            (lambda shape: torch.full(shape, 3.0, device="cuda"))
        if strided:
            x, z = _view(x, layout, pad), _view(z, layout, pad)
        c = torch.full((b, nc, D), 3.0, device="cuda").to(wl.torch_dtype)
        c32 = torch.full((b, nc, D), 3.0, device="cuda")
        dx, dz = mk((b, S, D)), mk((b, S, zc))
        dnw = torch.full((D,), 3.0, device="cuda") if epi else None
        if strided:
            csa.csa_compress_strided(dm, x, z, c, c32, **ep)
            csa.csa_compress_bwd_strided(dm, x, z, dc, dx, dz, dnorm_w=dnw, ws=ws, **ep)
        else:
            csa.csa_compress(dm, x, z, c, c32, **ep)
            csa.csa_compress_bwd(dm, x, z, dc, dx, dz, dnorm_w=dnw, ws=ws, **ep)
        torch.cuda.synchronize()
        return dict(c=c, c32=c32, dx=dx.contiguous(), dz=dz.contiguous(), dnw=dnw)

    ref, got = run(False), run(True)
    for k, v in ref.items():
        if v is None:
            continue
        assert torch.equal(got[k], v), f"{k}: strided compressor call differs from the contiguous call"
    assert bool((got["dx"][:, nc * wl.ratio:] == 0).all()) and bool((got["dz"][:, nc * wl.ratio:] == 0).all())


INDEX_CASES = [
    ("tiny_f32_sbhd", TINY.replace(b=2), "sbhd", 0, False),
    ("csa4_bf16_b2_sbhd", CSA4_SMALL.replace(b=2, sq=1030), "sbhd", 0, False),
    ("csa4_bf16_b3_pad", CSA4_SMALL.replace(b=3, sq=700, topk=64), "pad", 8, False),
    ("csa4_bf16_b2_sbhd_docs", CSA4_SMALL.replace(b=2, sq=900, topk=64), "sbhd", 0, True),
    ("one_head_unit_w_b2_sbhd", CSA4_SMALL.replace(b=2, sq=600, topk=64, idx_heads=1), "sbhd", 0, False),
]


@pytest.mark.parametrize("name,wl,layout,pad,docs", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_strided_indexer_matches_contiguous(gpu, name, wl, layout, pad, docs):
    """Sequence-major or padded q_i, k_i and w through csa_index_topk_strided
    (with and without packed documents): idx and score equal the contiguous
    call's exactly."""
    import compressed_sparse_attention_softmax_amd as csa
    say(f"[strided indexer] {name} b={wl.b} sq={wl.sq} hi={wl.idx_heads} di={wl.idx_dim} layout={layout}")
    inp = csa_synth.make_inputs(wl, 41, device="cuda", parts=("index",))
    dm = csa.dims_of(wl)
    b, S, kp = wl.b, wl.sq, wl.kprime
    doc = csa_synth.packed_doc_ids(b, S, 150.0, 43).cuda() if docs else None
    out = {}
    unit_w = name.startswith("one_head_unit_w")          # no w: unit weights
    for strided in (False, True):
        q_i, k_i, w = inp["q_i"], inp["k_i"], None if unit_w else inp["w"]
        idx = torch.full((b, S, kp), 7, dtype=torch.int32, device="cuda")
        score = torch.full((b, S, kp), 3.0, device="cuda")
        if strided:
            q_i, k_i = _view(q_i, layout, pad), _view(k_i, layout, pad)
            w = None if w is None else _view(w, layout, 4 if pad else 0)
            csa.csa_index_topk_strided(dm, q_i, k_i, w, idx, score, doc_ids=doc)
        else:
            csa.csa_index_topk(dm, q_i, k_i, w, idx, score, doc_ids=doc)
        torch.cuda.synchronize()
        out[strided] = (idx, score)
    assert torch.equal(out[True][0], out[False][0]), "idx: strided indexer call differs from the contiguous call"
    assert torch.equal(out[True][1], out[False][1]), "score: strided indexer call differs from the contiguous call"


@pytest.mark.parametrize("layout", ["pad", "sbhd"])
def test_strided_compressor_bwd_without_blocks_leaves_padding(gpu, layout):
    """sq < ratio (no compressed block): dx and dz are zero on every row of
    the view, and elements outside the view (padding) keep their values."""
    import compressed_sparse_attention_softmax_amd as csa
    wl = CSA4_SMALL.replace(b=2, sq=3)
    assert wl.n_c == 0
    say(f"[strided compressor, no block] layout={layout}")
    inp = csa_synth.make_inputs(wl, 47, device="cuda", parts=("compress",))
    dm = csa.dims_of(wl)
    b, S, D, zc = wl.b, wl.sq, wl.d, wl.z_channels
    x, z = _view(inp["x"], layout, 8), _view(inp["z"], layout, 8)
    dx = _empty_like_layout((b, S, D), torch.float32, layout, 8, fill=5.0)
    dz = _empty_like_layout((b, S, zc), torch.float32, layout, 8, fill=5.0)
    dc = torch.empty(b, 0, D, device="cuda")
    csa.csa_compress_bwd_strided(dm, x, z, dc, dx, dz)
    torch.cuda.synchronize()
    assert bool((dx == 0).all()) and bool((dz == 0).all())
    if layout == "pad":
        # the storage behind the views: the 8 padding columns of every row keep 5.0
        assert bool((dx.as_strided((b, S, D + 8), dx.stride())[..., D:] == 5.0).all())
        assert bool((dz.as_strided((b, S, zc + 8), dz.stride())[..., zc:] == 5.0).all())
