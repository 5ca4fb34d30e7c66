"""GPU parity of each hot-path step against the fp64 oracle, at sizes the
oracle finishes in seconds that still span several tiles and a ragged tail.

Every call goes through the C ABI (``libcsa.so``).  Inputs come from
``csa_synth``; expected values only from ``oracle``.  Each stage is fed the
same input values on both sides (stage isolation: the attention stage gets
an index list drawn by the input generator or computed by the oracle, never
one computed by the GPU).
"""
import os

import numpy as np
import pytest
import torch

import csa_synth
import oracle
from parity import check_close, check_topk_rows, f64, sample_rows, say, tol_of

pytestmark = pytest.mark.gpu

W = csa_synth.WORKLOADS
TINY = W["tiny_f32"]
# bf16 CSA-4 layer at reduced length: 1030 tokens (ragged vs ratio and tiles)
CSA4_SMALL = W["csa4_s4096"].replace(sq=1030, topk=96)
D512_SMALL = W["csa4_d512_s8192"].replace(sq=300, topk=40)
HCA_SMALL = W["hca128_s16384"].replace(sq=1100)


def dev(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def dims(wl, **kw):
    import compressed_sparse_attention_softmax_amd as csa
    return csa.dims_of(wl.replace(**kw) if kw else wl)


# ----------------------------------------------------------------- compressor
COMPRESS_CASES = [
    ("tiny_f32", TINY),
    ("csa4_bf16_overlap", CSA4_SMALL),
    ("csa4_bf16_rowscore", CSA4_SMALL.replace(z_channels=1)),
    ("d512_bf16", D512_SMALL),
    ("hca128_bf16", HCA_SMALL),
    ("f32_overlap_span12", TINY.replace(sq=203, span=12)),
    ("shorter_than_ratio", TINY.replace(sq=3)),
]


@pytest.mark.parametrize("name,wl", COMPRESS_CASES, ids=[c[0] for c in COMPRESS_CASES])
def test_compress_fwd_bwd(gpu, name, wl):
    csa = gpu
    say(f"[compress] {name} sq={wl.sq} d={wl.d} r={wl.ratio} L={wl.span} zc={wl.z_channels} {wl.dtype}")
    inp = csa_synth.make_inputs(wl, 11, device="cuda", parts=("compress",))
    dm = csa.dims_of(wl)
    b, S, D, nc = wl.b, wl.sq, wl.d, wl.n_c
    c = torch.empty(b, nc, D, dtype=wl.torch_dtype, device="cuda")
    c32 = torch.empty(b, nc, D, dtype=torch.float32, device="cuda")
    csa.csa_compress(dm, inp["x"], inp["z"], c, c32)
    g = torch.Generator(device="cuda").manual_seed(99)
    dc = torch.randn(b, nc, D, generator=g, device="cuda")
    dx = torch.full((b, S, D), 7.0, device="cuda")          # garbage: must be overwritten
    dz = torch.full((b, S, wl.z_channels), 7.0, device="cuda")
    csa.csa_compress_bwd(dm, inp["x"], inp["z"], dc, dx, dz)
    torch.cuda.synchronize()
    ref = oracle.compress(f64(inp["x"]), f64(inp["z"]), wl.ratio, wl.span)
    tol = tol_of(wl.torch_dtype)
    check_close("c32", c32, ref, tol)
    check_close("c", c, ref, tol)
    rdx, rdz = oracle.compress_bwd(f64(inp["x"]), f64(inp["z"]), f64(dc), wl.ratio, wl.span)
    check_close("dx", dx, rdx, tol)
    check_close("dz", dz, rdz, tol)


EPI_CASES = [
    ("tiny_f32_norm_rope_all", TINY, dict(norm=True, rope_dim=64)),
    ("tiny_f32_rope_only", TINY.replace(sq=203, span=12), dict(norm=False, rope_dim=16)),
    ("csa4_bf16_norm_rope64", CSA4_SMALL, dict(norm=True, rope_dim=64)),
    ("csa4_bf16_rowscore_norm", CSA4_SMALL.replace(z_channels=1), dict(norm=True, rope_dim=0)),
    ("csa4_bf16_frozen_norm_weight", CSA4_SMALL.replace(sq=500), dict(norm=True, rope_dim=64, want_dw=False)),
    ("d512_bf16_norm_rope64", D512_SMALL, dict(norm=True, rope_dim=64)),
    ("hca128_bf16_norm_rope64", HCA_SMALL, dict(norm=True, rope_dim=64)),
    ("shorter_than_ratio", TINY.replace(sq=3), dict(norm=True, rope_dim=8)),
]


@pytest.mark.parametrize("name,wl,kw", EPI_CASES, ids=[c[0] for c in EPI_CASES])
def test_compress_epilogue(gpu, name, wl, kw):
    from oracle import epilogue as ep
    csa = gpu
    say(f"[compress epilogue] {name} sq={wl.sq} d={wl.d} r={wl.ratio} L={wl.span} zc={wl.z_channels} {kw}")
    inp = csa_synth.make_inputs(wl, 13, device="cuda", parts=("compress",))
    dm = csa.dims_of(wl)
    b, S, D, nc = wl.b, wl.sq, wl.d, wl.n_c
    g = torch.Generator().manual_seed(17)
    nw = (1.0 + 0.2 * torch.randn(D, generator=g)) if kw["norm"] else None
    eps, rope, base = 1e-6, kw["rope_dim"], 40000.0
    epi = dict(norm_w=None if nw is None else nw.cuda(), norm_eps=eps, rope_dim=rope, rope_base=base)
    c = torch.empty(b, nc, D, dtype=wl.torch_dtype, device="cuda")
    c32 = torch.empty(b, nc, D, dtype=torch.float32, device="cuda")
    csa.csa_compress(dm, inp["x"], inp["z"], c, c32, **epi)
    dc = torch.randn(b, nc, D, generator=g).cuda()
    dx = torch.full((b, S, D), 7.0, device="cuda")
    dz = torch.full((b, S, wl.z_channels), 7.0, device="cuda")
    want_dw = kw.get("want_dw", True) and nw is not None
    dnw = torch.full((D,), 7.0, device="cuda") if want_dw else None
    ws = torch.empty(csa.csa_compress_bwd_workspace(dm), dtype=torch.uint8, device="cuda")
    csa.csa_compress_bwd(dm, inp["x"], inp["z"], dc, dx, dz, dnorm_w=dnw, ws=ws, **epi)
    torch.cuda.synchronize()
    x64, z64 = f64(inp["x"]), f64(inp["z"])
    pooled = oracle.compress(x64, z64, wl.ratio, wl.span)
    w64 = None if nw is None else nw.double().numpy()
    ref = ep.epilogue(pooled, w64, eps, rope, base)
    dy, rdw = ep.epilogue_bwd(pooled, w64, eps, rope, base, f64(dc))
    rdx, rdz = oracle.compress_bwd(x64, z64, dy, wl.ratio, wl.span)
    tol = tol_of(wl.torch_dtype)
    check_close("c32 (pooled, before the epilogue)", c32, pooled, tol)
    check_close("c", c, ref, tol)
    check_close("dx", dx, rdx, tol)
    check_close("dz", dz, rdz, tol)
    if want_dw:
        check_close("dnorm_w", dnw, rdw if nc > 0 else np.zeros(D), tol)


# ------------------------------------------------------------ indexer / top-k
def _index_case(wl, seed, rows=None, doc=None, **over):
    import compressed_sparse_attention_softmax_amd as csa
    inp = csa_synth.make_inputs(wl, seed, device="cuda", parts=("index",))
    inp.update({k: v for k, v in over.items()})
    dm = csa.dims_of(wl)
    kp = wl.kprime
    idx = torch.full((wl.b, wl.sq, kp), -7, dtype=torch.int32, device="cuda")
    sc = torch.empty(wl.b, wl.sq, kp, dtype=torch.float32, device="cuda")
    assert csa.csa_index_topk_workspace(dm) == 0
    csa.csa_index_topk(dm, inp["q_i"], inp["k_i"], inp["w"], idx, sc,
                       doc_ids=None if doc is None else doc.cuda())
    torch.cuda.synchronize()
    rows = oracle.all_rows(wl.b, wl.sq) if rows is None else rows
    rb, rt = torch.tensor(rows[:, 0]).cuda(), torch.tensor(rows[:, 1]).cuda()
    dnp = None if doc is None else doc.numpy()
    dense = oracle.index_scores(f64(inp["q_i"][rb, rt]), f64(inp["k_i"]), f64(inp["w"][rb, rt]), wl.ratio, rows,
                                dnp)
    oidx, _ = oracle.topk(dense, wl.ratio, wl.topk, rows, dnp)
    gi = idx[rb, rt].cpu().numpy()
    gs = sc[rb, rt].cpu().numpy()
    return gi, gs, oidx, dense, rows


# Cases with "rows": the oracle checks that many sampled query rows (always
# including the edges).  The sq = 32768 cases have n_c = 8192 blocks, more
# than the on-chip candidate buffer holds, so the streaming top-k runs its
# cut path (a buffer of 2 K' entries rounded to a tile, refilled and cut
# many times per row).
INDEX_CASES = [
    ("tiny_f32", TINY, None),
    ("csa4_bf16", CSA4_SMALL.replace(sq=1536), None),
    ("csa4_bf16_b2_ragged", CSA4_SMALL.replace(b=2, sq=1027, topk=50), None),
    ("streaming_cuts", CSA4_SMALL.replace(sq=32768, topk=100), 384),
    ("streaming_cuts_b2_ragged", CSA4_SMALL.replace(b=2, sq=32771, topk=130), 256),
    # n_c = 2048 with K' = 512: a 1024-entry buffer (two workgroups per CU)
    # rather than the whole prefix; K' = 2048, the largest, over n_c = 5003
    # with its 4096-entry buffer cut
    ("nc2048_kprime512", CSA4_SMALL.replace(sq=8192, topk=512), 384),
    ("kprime2048_cuts_b2_ragged", CSA4_SMALL.replace(b=2, sq=20013, topk=2048), 256),
    # K' >= ~200 leaves headroom for the loose cut (keep the K'-th best's bin
    # and above) before the exact one at the end
    ("kprime512_cuts", CSA4_SMALL.replace(sq=32768, topk=512), 384),
    ("idx_dim64_heads40", CSA4_SMALL.replace(idx_heads=40, idx_dim=64, sq=900, topk=70), None),
    # fp32 at d_i = 128 (the cut reads its buffer one entry per lane at a time)
    ("f32_idx_dim128_heads20", TINY.replace(idx_heads=20, idx_dim=128, sq=700, topk=40), None),
    ("f32_idx_dim128_cuts", TINY.replace(idx_heads=20, idx_dim=128, sq=16001, topk=30), 256),
    ("one_block", CSA4_SMALL.replace(sq=5, topk=40), None),
    ("b3_sq9", CSA4_SMALL.replace(b=3, sq=9, topk=1), None),
]


def _edge_rows(wl, n, seed):
    kp, r = wl.kprime, wl.ratio
    must = [0, 1, r - 1, r, kp * r - 2, kp * r - 1, kp * r, 2 * kp * r, wl.sq // 2, wl.sq - 2, wl.sq - 1]
    return sample_rows(wl.b, wl.sq, n, seed, must)


@pytest.mark.parametrize("name,wl,nrows", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_index_topk(gpu, name, wl, nrows):
    say(f"[index_topk] {name} b={wl.b} sq={wl.sq} HI={wl.idx_heads} DI={wl.idx_dim} K={wl.topk} rows={nrows}")
    rows = None if nrows is None else _edge_rows(wl, nrows, 21)
    gi, gs, oidx, dense, rows = _index_case(wl, 21, rows=rows)
    exact = check_topk_rows(gi, gs, oidx, dense, rows[:, 1], wl.ratio, wl.n_c, wl.kprime,
                            score_tol=tol_of(wl.torch_dtype))
    say(f"  rows identical to the oracle: {exact}/{len(rows)}")


@pytest.mark.parametrize("heads,topk", [(8, 40), (64, 1024)])
def test_index_topk_exact_integer_scores_and_ties(gpu, heads, topk):
    # small integer inputs make every fp32 score exact, so the GPU must match
    # the oracle bit for bit, including the lowest-index rule on exact ties;
    # n_c = 8192 blocks drive the streaming cut path (with 64 heads and
    # K' = 1024, 2048-entry buffers)
    say(f"[index_topk exact] heads={heads} K={topk}")
    wl = CSA4_SMALL.replace(sq=32768, topk=topk, idx_heads=heads)
    g = torch.Generator().manual_seed(5)
    qi = torch.randint(-2, 3, (1, wl.sq, heads, 128), generator=g).to(torch.bfloat16)
    ki = torch.randint(-1, 2, (1, wl.n_c, 128), generator=g).to(torch.bfloat16)
    ki[0, 100:140] = ki[0, 7]                                   # many identical keys
    ki[0, 5000:5100] = ki[0, 4000]
    w = (torch.randint(-2, 5, (1, wl.sq, heads), generator=g).float() / 4)
    rows = _edge_rows(wl, 512, 0)
    gi, gs, oidx, dense, rows = _index_case(wl, 0, rows=rows, q_i=qi.cuda(), k_i=ki.cuda(), w=w.cuda())
    np.testing.assert_array_equal(gi, oidx)
    np.testing.assert_array_equal(gs[gi >= 0], dense[np.nonzero(gi >= 0)[0], gi[gi >= 0]])


DOC_INDEX_CASES = [
    ("tiny_f32", TINY.replace(b=2, sq=301), 40, None),
    ("csa4_bf16_b2", CSA4_SMALL.replace(b=2, sq=1500, topk=60), 300, None),
    ("csa4_bf16_short_docs", CSA4_SMALL.replace(sq=1200, topk=40), 30, None),
    ("csa4_bf16_streaming_cuts", CSA4_SMALL.replace(sq=32768, topk=64), 2000, 256),
    ("csa4_bf16_nc2048", CSA4_SMALL.replace(sq=8192, topk=300), 1500, 256),
    ("csa4_bf16_kprime512_cuts", CSA4_SMALL.replace(sq=32768, topk=512), 2000, 256),
]


@pytest.mark.parametrize("name,wl,mean,nrows", DOC_INDEX_CASES, ids=[c[0] for c in DOC_INDEX_CASES])
def test_index_topk_packed_documents(gpu, name, wl, mean, nrows):
    say(f"[index_topk docs] {name} b={wl.b} sq={wl.sq} K={wl.topk} mean doc length {mean} rows={nrows}")
    doc = csa_synth.packed_doc_ids(wl.b, wl.sq, mean, 7)
    rows = None if nrows is None else _edge_rows(wl, nrows, 23)
    gi, gs, oidx, dense, rows = _index_case(wl, 23, rows=rows, doc=doc)
    exact = check_topk_rows(gi, gs, oidx, dense, rows[:, 1], wl.ratio, wl.n_c, wl.kprime,
                            score_tol=tol_of(wl.torch_dtype), docs=True)
    say(f"  rows identical to the oracle: {exact}/{len(rows)}")


@pytest.mark.parametrize("sq,topk,nrows", [(600, 30, None), (32768, 512, 256)])
def test_index_topk_all_zero_keys(gpu, sq, topk, nrows):
    # every score 0: the lowest indices win; at sq 32768 with K' = 512 every
    # mid-stream cut finds an empty score range, so the room-making cut gives
    # way to the exact one
    say(f"[index_topk zero keys] sq={sq} K={topk}")
    wl = CSA4_SMALL.replace(sq=sq, topk=topk)
    ki = torch.zeros(1, wl.n_c, 128, dtype=torch.bfloat16, device="cuda")
    rows = None if nrows is None else _edge_rows(wl, nrows, 3)
    gi, gs, oidx, dense, rows = _index_case(wl, 3, rows=rows, k_i=ki)
    np.testing.assert_array_equal(gi, oidx)
    assert np.all(gs[gi >= 0] == 0.0) and not np.any(np.signbit(gs[gi >= 0]))


# ------------------------------------------------------------------ attention
def _attn_case(wl, seed, idx_mode="random", with_sink=True, window_only=False, junk=False, dsink_only=False,
               doc_len=None):
    import compressed_sparse_attention_softmax_amd as csa
    inp = csa_synth.make_inputs(wl, seed, device="cuda", parts=("attn", "compress", "bwd"),
                                with_sink=with_sink)
    b, S, H, D, nc = wl.b, wl.sq, wl.h, wl.d, wl.n_c
    doc = None if doc_len is None else csa_synth.packed_doc_ids(b, S, doc_len, seed + 2)
    docn = None if doc is None else doc.numpy()
    docg = None if doc is None else doc.cuda()
    # compressed rows: the oracle's pooling, cast once to the working dtype
    c = None
    if not window_only:
        c64 = oracle.compress(f64(inp["x"]), f64(inp["z"]), wl.ratio, wl.span)
        c = torch.tensor(c64).to(wl.torch_dtype).cuda()
    idx = None
    if not window_only and idx_mode != "dense":
        if idx_mode == "random":
            idx = csa_synth.random_topk_indices(wl, seed + 1)
        elif idx_mode == "indexer":      # the oracle indexer's selection (document-aware)
            ii = csa_synth.make_inputs(wl, seed + 3, parts=("index",))
            oi, _, _ = oracle.index_topk(f64(ii["q_i"]), f64(ii["k_i"]), f64(ii["w"]), wl.ratio, wl.topk,
                                         doc=docn)
            idx = torch.tensor(oi).reshape(b, S, wl.kprime)
        elif idx_mode == "block0":
            idx = torch.full((b, S, wl.kprime), -1, dtype=torch.int32)
            idx[:, wl.ratio - 1:, 0] = 0
        if junk:
            g = torch.Generator().manual_seed(seed)
            idx = idx.clone()
            kp = wl.kprime
            for bi in range(b):
                for t in range(0, S, 3):
                    nv = (t + 1) // wl.ratio
                    if kp >= 3 and nv >= 2:
                        idx[bi, t, 1] = idx[bi, t, 0]               # duplicate within a row
                        idx[bi, t, 2] = -1                          # hole in the middle
                    if kp >= 1:
                        idx[bi, t, kp - 1] = nv + int(torch.randint(0, 5, (1,), generator=g))  # not yet valid
        idx = idx.cuda()
    dm = csa.dims_of(wl)
    dtype = wl.torch_dtype
    out = torch.empty(b, S, H, D, dtype=dtype, device="cuda")
    lse = torch.empty(b, S, H, dtype=torch.float32, device="cuda")
    csa.csa_sparse_attn_fwd(dm, inp["q"], inp["kv"], c, idx, inp["sink"], wl.scale, out, lse, doc_ids=docg)
    dq = torch.empty_like(out)
    dkv = torch.full((b, S, D), 3.0, device="cuda")
    dc = torch.full((b, nc, D), 3.0, device="cuda") if c is not None else None
    dsink = torch.full((H,), 3.0, device="cuda") if with_sink else None
    ws = torch.empty(csa.csa_sparse_attn_bwd_workspace(dm), dtype=torch.uint8, device="cuda")
    if dsink_only:       # gradient gate closed: only dsink is produced
        dq = dkv = dc = None
    csa.csa_sparse_attn_bwd(dm, inp["q"], inp["kv"], c, idx, inp["sink"], wl.scale, out, lse, inp["do"],
                            dq, dkv, dc, dsink, ws=ws, doc_ids=docg)
    torch.cuda.synchronize()
    rows = oracle.all_rows(b, S)
    q = f64(inp["q"]).reshape(b * S, H, D)
    kv = f64(inp["kv"])
    cc = f64(c) if c is not None else np.zeros((b, 0, D))
    ii = None if idx is None else idx.cpu().numpy().reshape(b * S, -1)
    sink = None if inp["sink"] is None else f64(inp["sink"])
    window = wl.window
    ratio = wl.ratio
    ro, rl = oracle.attn_fwd(q, kv, cc, ii, sink, wl.scale, window, ratio, rows, doc=docn)
    rdq, rdkv, rdc, rds = oracle.attn_bwd(q, kv, cc, ii, sink, wl.scale, window, ratio, rows,
                                          f64(inp["do"]).reshape(b * S, H, D), doc=docn)
    tol = tol_of(dtype)
    check_close("out", out.reshape(b * S, H, D), ro, tol)
    check_close("lse", lse.reshape(b * S, H), rl, tol)
    if not dsink_only:
        check_close("dq", dq.reshape(b * S, H, D), rdq, tol)
        check_close("dkv", dkv, rdkv, tol)
    if dc is not None:
        check_close("dc", dc, rdc, tol)
    if dsink is not None:
        check_close("dsink", dsink, rds, tol)


ATTN_CASES = [
    ("tiny_f32", TINY, {}),
    ("tiny_f32_nosink", TINY, dict(with_sink=False)),
    ("tiny_f32_window1", TINY.replace(window=1), {}),
    ("tiny_f32_junk_idx", TINY, dict(junk=True)),
    ("csa4_bf16", CSA4_SMALL.replace(sq=640), {}),
    ("csa4_bf16_b2_h48", CSA4_SMALL.replace(b=2, sq=333, h=48, topk=40), {}),
    ("csa4_bf16_junk_idx", CSA4_SMALL.replace(sq=400, topk=40), dict(junk=True)),
    ("csa4_bf16_block0_repeat", CSA4_SMALL.replace(sq=700, topk=8), dict(idx_mode="block0")),
    ("csa4_bf16_dense", CSA4_SMALL.replace(sq=500), dict(idx_mode="dense")),
    ("csa4_bf16_window_only", CSA4_SMALL.replace(sq=300), dict(window_only=True)),
    ("csa4_bf16_dsink_only", CSA4_SMALL.replace(sq=300), dict(dsink_only=True)),
    ("tiny_f32_docs_dense", TINY.replace(b=2, sq=257), dict(idx_mode="dense", doc_len=30)),
    ("tiny_f32_docs_indexer", TINY.replace(b=2, sq=257), dict(idx_mode="indexer", doc_len=30)),
    ("csa4_bf16_docs_indexer", CSA4_SMALL.replace(b=2, sq=700, topk=40), dict(idx_mode="indexer", doc_len=150)),
    ("csa4_bf16_docs_random_idx", CSA4_SMALL.replace(sq=500, topk=40), dict(doc_len=100)),
    ("csa4_bf16_docs_dense", CSA4_SMALL.replace(sq=600), dict(idx_mode="dense", doc_len=90)),
    ("csa4_bf16_docs_window_only", CSA4_SMALL.replace(sq=400), dict(window_only=True, doc_len=60)),
    ("csa4_bf16_docs_h48", CSA4_SMALL.replace(b=2, sq=333, h=48, topk=40), dict(idx_mode="indexer", doc_len=70)),
    ("d512_bf16_docs", D512_SMALL, dict(idx_mode="indexer", doc_len=80)),
    # no sink, short documents: the first row chunks of many windows lie
    # wholly in an earlier document (every logit of the chunk masked)
    ("csa4_bf16_docs_nosink", CSA4_SMALL.replace(b=2, sq=500, topk=40),
     dict(idx_mode="indexer", doc_len=40, with_sink=False)),
    ("csa4_bf16_docs_window_only_nosink", CSA4_SMALL.replace(sq=400),
     dict(window_only=True, doc_len=40, with_sink=False)),
    ("d512_bf16", D512_SMALL, {}),
    # d = 512 stages 32 heads per unit of the key-stationary loop: a second
    # unit that is partly padding (48 heads) or wholly padding (20 heads)
    ("d512_bf16_h48", D512_SMALL.replace(sq=200, h=48), {}),
    ("d512_bf16_h20_b2", D512_SMALL.replace(b=2, sq=150, h=20), {}),
    ("hca128_bf16_dense", HCA_SMALL, dict(idx_mode="dense")),
    # degenerate lengths: one token; shorter than the ratio (no compressed
    # row at all, the zero-size tensors arrive as NULL); one compressed row
    ("tiny_f32_sq1", TINY.replace(sq=1), {}),
    ("csa4_bf16_shorter_than_ratio", CSA4_SMALL.replace(sq=3), {}),
    ("csa4_bf16_sq1_window_only", CSA4_SMALL.replace(sq=1), dict(window_only=True)),
    ("csa4_bf16_sq5_dense", CSA4_SMALL.replace(sq=5), dict(idx_mode="dense")),
    ("csa4_bf16_b3_sq9", CSA4_SMALL.replace(b=3, sq=9, topk=2), {}),
    # head counts that leave head slots of the 16-wide tiles empty: one
    # head, one past 32, and 17 heads at d = 64
    ("csa4_bf16_h1", CSA4_SMALL.replace(sq=300, h=1, topk=40), {}),
    ("csa4_bf16_h33", CSA4_SMALL.replace(sq=300, h=33, topk=40), {}),
    ("bf16_d64_h17", CSA4_SMALL.replace(sq=300, h=17, d=64, z_channels=64, topk=40), {}),
    ("tiny_f32_h5", TINY.replace(h=5), {}),
]


@pytest.mark.parametrize("name,wl,kw", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_sparse_attention_fwd_bwd(gpu, name, wl, kw):
    say(f"[attn] {name} b={wl.b} sq={wl.sq} h={wl.h} d={wl.d} W={wl.window} r={wl.ratio} K={wl.topk} {kw}")
    _attn_case(wl, 31, **kw)


# ------------------------------------------------ indexer distillation loss
def _loss_case(wl, seed, junk=False, grads=True):
    import compressed_sparse_attention_softmax_amd as csa
    from oracle import indexer_loss as il
    inp = csa_synth.make_inputs(wl, seed, device="cpu", parts=("attn", "compress", "index"))
    b, S, H, D, nc, kp = wl.b, wl.sq, wl.h, wl.d, wl.n_c, wl.kprime
    dt = wl.torch_dtype
    c = torch.tensor(oracle.compress(f64(inp["x"]), f64(inp["z"]), wl.ratio, wl.span)).to(dt)
    qi, ki, w = f64(inp["q_i"]), f64(inp["k_i"]), f64(inp["w"])
    oidx, osc, _ = oracle.index_topk(qi, ki, w, wl.ratio, wl.topk)
    idx = np.asarray(oidx, dtype=np.int32).reshape(b * S, kp).copy()
    score = np.asarray(osc, dtype=np.float32).reshape(b * S, kp).copy()
    if junk:
        g = np.random.default_rng(seed)
        for n in range(0, b * S, 3):
            t = n % S
            nv = min((t + 1) // wl.ratio, nc)
            if kp >= 3 and nv >= 3:
                idx[n, 1] = -1                                   # hole
                idx[n, 2] = nv + int(g.integers(0, 4))           # not yet valid
    rows = oracle.all_rows(b, S)
    q64 = f64(inp["q"]).reshape(b * S, H, D)
    _, lse64 = oracle.attn_fwd(q64, f64(inp["kv"]), f64(c), idx, f64(inp["sink"]), wl.scale, wl.window,
                               wl.ratio, rows)
    lse = torch.tensor(lse64, dtype=torch.float32)               # the stage input, rounded once
    gen = torch.Generator().manual_seed(seed + 5)
    dkl = torch.randn(b, S, generator=gen)
    dm = csa.dims_of(wl)
    cu = lambda a: torch.as_tensor(a).cuda()
    kl = torch.full((b, S), 7.0, device="cuda")
    out = {}
    if grads:
        out = dict(dq_i=torch.full((b, S, wl.idx_heads, wl.idx_dim), 7.0, dtype=dt, device="cuda"),
                   dw=torch.full((b, S, wl.idx_heads), 7.0, device="cuda"),
                   dk_i=torch.full((b, nc, wl.idx_dim), 7.0, device="cuda"))
        ws = torch.empty(csa.csa_indexer_loss_workspace(dm), dtype=torch.uint8, device="cuda")
    else:
        ws = None
    csa.csa_indexer_loss(dm, cu(inp["q"]), cu(c), cu(lse.reshape(b, S, H)), cu(inp["q_i"]), cu(inp["k_i"]),
                         cu(inp["w"]), cu(idx.reshape(b, S, kp)), cu(score.reshape(b, S, kp)), wl.scale, kl=kl,
                         dkl=cu(dkl) if grads else None, ws=ws, **out)
    torch.cuda.synchronize()
    # oracle, fed the same rounded values
    nv = np.minimum((rows[:, 1] + 1) // wl.ratio, nc)
    valid = (idx >= 0) & (idx < nv[:, None])
    target = il.teacher_target(q64, f64(c), f64(lse), idx, wl.scale, wl.ratio, rows)
    r_kl, predict = il.kl_loss(target, np.where(valid, score.astype(np.float64), -np.inf))
    tol = tol_of(dt)
    check_close("kl", kl.reshape(-1), r_kl, tol)
    if grads:
        rdq, rdw, rdk, _ = il.loss_bwd(qi.reshape(b * S, wl.idx_heads, wl.idx_dim), ki,
                                       w.reshape(b * S, wl.idx_heads), idx, wl.ratio, rows, target, predict,
                                       dkl.double().numpy().reshape(-1))
        check_close("dq_i", out["dq_i"].reshape(b * S, wl.idx_heads, wl.idx_dim), rdq, tol)
        check_close("dw", out["dw"].reshape(b * S, wl.idx_heads), rdw, tol)
        check_close("dk_i", out["dk_i"], rdk, tol)


LOSS_CASES = [
    ("tiny_f32", TINY, {}),
    ("tiny_f32_b2_junk_idx", TINY.replace(b=2, sq=203), dict(junk=True)),
    ("tiny_f32_kl_only", TINY, dict(grads=False)),
    ("csa4_bf16", CSA4_SMALL, {}),
    ("csa4_bf16_k512", CSA4_SMALL.replace(sq=2100, topk=512), {}),
    ("csa4_bf16_b2_h48_junk", CSA4_SMALL.replace(b=2, sq=333, h=48, topk=40), dict(junk=True)),
    ("idx_dim64_heads40", CSA4_SMALL.replace(idx_heads=40, idx_dim=64, sq=900, topk=70), {}),
    ("d512_bf16", D512_SMALL, {}),
    ("shorter_than_ratio", TINY.replace(sq=3), {}),
]


@pytest.mark.parametrize("name,wl,kw", LOSS_CASES, ids=[c[0] for c in LOSS_CASES])
def test_indexer_loss(gpu, name, wl, kw):
    say(f"[indexer_loss] {name} b={wl.b} sq={wl.sq} h={wl.h} d={wl.d} HI={wl.idx_heads} DI={wl.idx_dim} "
        f"K={wl.topk} {kw}")
    _loss_case(wl, 41, **kw)


# ------------------------------------------ simplified DSA over GQA
GQA = csa_synth.GQA_WORKLOADS


def _gqa_indices(wl, inp, junk=False):
    """The oracle's one-head, unit-weight, ratio-1 selection [b, sq, K']."""
    b, S = wl.b, wl.sq
    idx, _, _ = oracle.index_topk(f64(inp["q_i"]), f64(inp["k_i"]), np.ones((b, S, 1)), 1, wl.topk)
    idx = np.asarray(idx, dtype=np.int32).reshape(b, S, wl.kprime).copy()
    if junk == "one":
        idx[:, 40, 1] = idx[:, 40, 0]                            # one repeat: its stack scans the index rows
    elif junk:
        idx[:, 3::5, 1] = idx[:, 3::5, 0]                        # repeated entry
        idx[:, 7, :] = -1                                        # a query with no valid slot
        idx[:, 11::7, -1] = np.minimum(np.arange(11, S, 7) + 3, S - 1)[None, :]   # not yet valid
    return idx


def test_index_topk_simplified_one_head(gpu):
    import compressed_sparse_attention_softmax_amd as csa
    wl = GQA["dsa_gqa_tiny_f32"].replace(sq=700, topk=60, dtype="bf16", idx_dim=128)
    say(f"[index_topk simplified] sq={wl.sq} K={wl.topk} DI={wl.idx_dim}")
    inp = csa_synth.make_gqa_inputs(wl, 3, device="cuda")
    dm = csa.make_dims(wl.b, wl.sq, ratio=1, idx_heads=1, idx_dim=wl.idx_dim, topk=wl.topk)
    idx = torch.full((wl.b, wl.sq, wl.kprime), -7, dtype=torch.int32, device="cuda")
    sc = torch.empty(wl.b, wl.sq, wl.kprime, device="cuda")
    csa.csa_index_topk(dm, inp["q_i"], inp["k_i"], None, idx, sc)
    torch.cuda.synchronize()
    rows = oracle.all_rows(wl.b, wl.sq)
    oidx, _, dense = oracle.index_topk(f64(inp["q_i"]), f64(inp["k_i"]), np.ones((wl.b, wl.sq, 1)), 1, wl.topk,
                                       rows=rows)
    exact = check_topk_rows(idx.cpu().numpy().reshape(-1, wl.kprime), sc.cpu().numpy().reshape(-1, wl.kprime),
                            oidx, dense, rows[:, 1], 1, wl.sq, wl.kprime, score_tol=tol_of(torch.bfloat16))
    say(f"  rows identical to the oracle: {exact}/{len(rows)}")


GQA_CASES = [
    ("tiny_f32_dp64", GQA["dsa_gqa_tiny_f32"], {}),
    ("tiny_f32_junk_idx", GQA["dsa_gqa_tiny_f32"].replace(b=1, sq=150), dict(junk=True)),
    ("bf16_dp128_g4", GQA["dsa_gqa_s4096"].replace(sq=700, h=16, h_kv=4, d_qk=64, d_v=64, topk=64), {}),
    ("bf16_dp256_g4", GQA["dsa_gqa_s4096"].replace(sq=600, topk=128), {}),
    ("bf16_dp256_g16_junk", GQA["dsa_gqa_s4096"].replace(sq=333, h=32, h_kv=2, topk=40), dict(junk=True)),
    ("bf16_dp512_mqa", GQA["dsa_gqa_s4096"].replace(sq=300, h=8, h_kv=1, d_qk=192, d_v=320, topk=50), {}),
    ("bf16_dp64", GQA["dsa_gqa_s4096"].replace(sq=257, h=8, h_kv=2, d_qk=32, d_v=32, topk=30), {}),
    ("f32_dp128", GQA["dsa_gqa_tiny_f32"].replace(sq=190, d_qk=64, d_v=64), {}),
    ("bf16_dp256_one_head_per_group", GQA["dsa_gqa_s4096"].replace(sq=260, h=8, h_kv=8, topk=33), {}),
    ("bf16_dp256_unequal_halves", GQA["dsa_gqa_s4096"].replace(sq=211, h=16, h_kv=4, d_qk=96, d_v=160, topk=40), {}),
    ("bf16_dp256_g4_one_repeat", GQA["dsa_gqa_s4096"].replace(sq=400, h=8, h_kv=2, topk=64), dict(junk="one")),
    # q starts 2 bytes past an alignment boundary: the packing copies single elements
    ("bf16_dp128_misaligned_q", GQA["dsa_gqa_s4096"].replace(sq=300, h=8, h_kv=2, d_qk=64, d_v=64, topk=40),
     dict(misalign=True)),
]


@pytest.mark.parametrize("name,wl,kw", GQA_CASES, ids=[c[0] for c in GQA_CASES])
def test_dsa_gqa_fwd_bwd(gpu, name, wl, kw):
    import compressed_sparse_attention_softmax_amd as csa
    from oracle import dsa_gqa
    say(f"[dsa gqa] {name} b={wl.b} sq={wl.sq} h={wl.h} h_kv={wl.h_kv} d_qk={wl.d_qk} d_v={wl.d_v} "
        f"K={wl.topk} {wl.dtype} {kw}")
    inp = csa_synth.make_gqa_inputs(wl, 29, device="cuda")
    idx = _gqa_indices(wl, inp, junk=kw.get("junk", False))
    if kw.get("misalign"):
        qm = torch.empty(inp["q"].numel() + 1, dtype=inp["q"].dtype, device="cuda")[1:].view(inp["q"].shape)
        qm.copy_(inp["q"])
        assert qm.data_ptr() % 16 != 0
        inp["q"] = qm
    g = csa.csa_gqa_dims(wl.b, wl.sq, wl.h, wl.h_kv, wl.d_qk, wl.d_v, wl.topk)
    dt = wl.torch_dtype
    b, S = wl.b, wl.sq
    out = torch.full((b, S, wl.h, wl.d_v), 7.0, dtype=dt, device="cuda")
    lse = torch.full((b, S, wl.h), 7.0, device="cuda")
    ws = torch.empty(csa.csa_dsa_gqa_workspace(g, dt, True), dtype=torch.uint8, device="cuda")
    idx_d = torch.tensor(idx).cuda()
    csa.csa_dsa_gqa_fwd(g, inp["q"], inp["k"], inp["v"], idx_d, wl.scale, out, lse, ws)
    dq = torch.full_like(inp["q"], 7.0)
    dk = torch.full((b, S, wl.h_kv, wl.d_qk), 7.0, device="cuda")
    dv = torch.full((b, S, wl.h_kv, wl.d_v), 7.0, device="cuda")
    csa.csa_dsa_gqa_bwd(g, inp["q"], inp["k"], inp["v"], idx_d, wl.scale, out, lse, inp["do"], dq, dk, dv, ws)
    torch.cuda.synchronize()
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    ro, rl = dsa_gqa.fwd(q, k, v, idx, wl.scale)
    tol = tol_of(dt)
    check_close("out", out, ro, tol)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse.cpu().numpy()), empty)
    check_close("lse", lse.cpu().numpy()[~empty], rl[~empty], tol)
    # the backward is fed the forward's own (rounded) output, as a caller would
    rdq, rdk, rdv = dsa_gqa.bwd(q, k, v, idx, wl.scale, f64(out), np.where(empty, -np.inf, f64(lse)), do)
    check_close("dq", dq, rdq, tol)
    check_close("dk", dk, rdk, tol)
    check_close("dv", dv, rdv, tol)


def test_indexer_loss_dense_warmup_by_composition(gpu):
    """The dense warm-up form of the distillation loss (teacher and student
    over every valid block, not only the selected ones) composed from the
    entry points: the indexer with K' = n_c returns every valid block and its
    score, the attention's dense mode returns the dense LSE, and the loss
    takes both."""
    import compressed_sparse_attention_softmax_amd as csa
    from oracle import indexer_loss as il
    wl = CSA4_SMALL.replace(sq=700)
    wl = wl.replace(topk=wl.n_c)
    say(f"[indexer_loss dense warm-up] sq={wl.sq} n_c={wl.n_c}")
    inp = csa_synth.make_inputs(wl, 43, device="cuda", parts=("attn", "compress", "index"))
    b, S, H, D, nc = wl.b, wl.sq, wl.h, wl.d, wl.n_c
    dm = csa.dims_of(wl)
    c = torch.tensor(oracle.compress(f64(inp["x"]), f64(inp["z"]), wl.ratio, wl.span)).to(wl.torch_dtype).cuda()
    idx = torch.empty(b, S, nc, dtype=torch.int32, device="cuda")
    sc = torch.empty(b, S, nc, device="cuda")
    csa.csa_index_topk(dm, inp["q_i"], inp["k_i"], inp["w"], idx, sc)
    out = torch.empty(b, S, H, D, dtype=wl.torch_dtype, device="cuda")
    lse = torch.empty(b, S, H, device="cuda")
    csa.csa_sparse_attn_fwd(dm, inp["q"], inp["kv"], c, None, inp["sink"], wl.scale, out, lse)
    kl = torch.empty(b, S, device="cuda")
    dkl = torch.ones(b, S, device="cuda")
    dq_i = torch.empty_like(inp["q_i"])
    dw = torch.empty(b, S, wl.idx_heads, device="cuda")
    dk_i = torch.empty(b, nc, wl.idx_dim, device="cuda")
    ws = torch.empty(csa.csa_indexer_loss_workspace(dm), dtype=torch.uint8, device="cuda")
    csa.csa_indexer_loss(dm, inp["q"], c, lse, inp["q_i"], inp["k_i"], inp["w"], idx, sc, wl.scale, kl=kl, dkl=dkl,
                         dq_i=dq_i, dw=dw, dk_i=dk_i, ws=ws)
    torch.cuda.synchronize()
    rows = oracle.all_rows(b, S)
    # every valid block, in order: exactly what the indexer must return at K' = n_c
    nv = np.minimum((rows[:, 1] + 1) // wl.ratio, nc)
    full = np.where(np.arange(nc)[None, :] < nv[:, None], np.arange(nc)[None, :], -1).astype(np.int32)
    np.testing.assert_array_equal(idx.cpu().numpy().reshape(-1, nc), full)
    q64 = f64(inp["q"]).reshape(b * S, H, D)
    _, rl = oracle.attn_fwd(q64, f64(inp["kv"]), f64(c), None, f64(inp["sink"]), wl.scale, wl.window, wl.ratio, rows)
    qi, w = f64(inp["q_i"]).reshape(b * S, wl.idx_heads, wl.idx_dim), f64(inp["w"]).reshape(b * S, wl.idx_heads)
    got = il.indexer_loss(q64, f64(c), rl, qi, f64(inp["k_i"]), w, full, wl.scale, wl.ratio, rows, dkl=np.ones(b * S))
    tol = tol_of(wl.torch_dtype)
    check_close("kl", kl.reshape(-1), got["kl"], tol)
    check_close("dq_i", dq_i.reshape(b * S, wl.idx_heads, wl.idx_dim), got["dq_i"], tol)
    check_close("dw", dw.reshape(b * S, wl.idx_heads), got["dw"], tol)
    check_close("dk_i", dk_i, got["dk_i"], tol)
