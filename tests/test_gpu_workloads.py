"""Parity at the five full workload sizes, in the launch configuration the
benchmark times (one pass of ``pipeline.forward`` / ``pipeline.backward``).

* compressor forward: every output row;
* indexer + top-k: sampled query rows (edge positions plus random ones), with
  the near-tie band rule;
* attention forward: every sampled row, the oracle fed the GPU's own index
  rows (so a forward error is never hidden behind a top-k difference);
* attention backward: the backward is linear in dO, so a dO that is zero
  except on chosen rows makes every gradient (dq rows, all of dkv, dc,
  dsink) computable by the oracle from those rows alone.  The rows are
  stratified: one in every block of consecutive queries that the backward
  reduces as a unit (csa_sparse_attn_bwd_query_block), in every batch row,
  so every block contributes gradient;
* compressor backward: chained from each side's own dc.
"""
import numpy as np
import pytest
import torch

import csa_synth
import oracle
from parity import check_close, check_topk_rows, f64, sample_rows, say, tol_of

pytestmark = pytest.mark.gpu

N_ROWS = {"tiny_f32": 256, "csa4_s4096": 96, "csa4_d512_s8192": 48, "hca128_s16384": 48,
          "csa4_s65536_skew": 40}
N_BWD_ROWS = {"tiny_f32": 256, "csa4_s4096": 48, "csa4_d512_s8192": 24, "hca128_s16384": 24,
              "csa4_s65536_skew": 24}


@pytest.mark.parametrize("name", csa_synth.WORKLOAD_ORDER)
def test_workload_parity(gpu, name):
    _whole_pass(csa_synth.WORKLOADS[name], csa_synth.WORKLOAD_SEEDS[name], N_ROWS[name], N_BWD_ROWS[name])


# the largest index rows the kernels take (K' = 2048) with the widest rows
# (d = 512): the largest LDS footprint of the query kernels (two 32-row
# tiles of 1 KiB rows plus the index row) and of the indexer's candidate buffer
MAX_CASES = [
    ("d512_topk2048", csa_synth.WORKLOADS["csa4_d512_s8192"].replace(sq=8300, topk=2048), 16, 8),
]


@pytest.mark.parametrize("name,wl,nf,nb", MAX_CASES, ids=[c[0] for c in MAX_CASES])
def test_maximum_sizes(gpu, name, wl, nf, nb):
    _whole_pass(wl, 17, nf, nb)


# the shortest sequences: one token, shorter than the ratio (no compressed
# row: the indexer has nothing to select and the attention sees the window
# only), and one compressed row, in the bench's and the fp32 configuration
MIN_CASES = [
    ("csa4_sq1", csa_synth.WORKLOADS["csa4_s4096"].replace(sq=1)),
    ("csa4_sq3", csa_synth.WORKLOADS["csa4_s4096"].replace(sq=3)),
    ("csa4_sq5", csa_synth.WORKLOADS["csa4_s4096"].replace(sq=5)),
    ("tiny_f32_sq3_b2", csa_synth.WORKLOADS["tiny_f32"].replace(b=2, sq=3)),
]


@pytest.mark.parametrize("name,wl", MIN_CASES, ids=[c[0] for c in MIN_CASES])
def test_minimum_sizes(gpu, name, wl):
    _whole_pass(wl, 19, 16, 16)


def _block_rows(b, S, qb, seed, extra):
    """One random query of every block [k*qb, (k+1)*qb) of every batch row,
    the last query of each batch row, and `extra` more random rows."""
    rng = np.random.default_rng(seed + 101)
    rows = set()
    for bi in range(b):
        for t0 in range(0, S, qb):
            rows.add((bi, int(rng.integers(t0, min(S, t0 + qb)))))
        rows.add((bi, S - 1))
    for _ in range(extra):
        rows.add((int(rng.integers(b)), int(rng.integers(S))))
    return np.array(sorted(rows), dtype=np.int64)


def _whole_pass(wl, seed, n_rows, n_bwd_rows):
    import compressed_sparse_attention_softmax_amd as csa
    from compressed_sparse_attention_softmax_amd import pipeline
    name = wl.name
    say(f"[workload] {name} seed={seed} b={wl.b} sq={wl.sq} h={wl.h} d={wl.d} r={wl.ratio} "
        f"L={wl.span} W={wl.window} K={wl.topk} {wl.dtype}")
    torch.cuda.empty_cache()
    inp = csa_synth.make_inputs(wl, seed, device="cuda")
    dm = csa.dims_of(wl)
    buf = pipeline.allocate(dm, wl.torch_dtype, wl.z_channels)
    pipeline.forward(dm, inp, buf, wl.scale)
    torch.cuda.synchronize()
    tol = tol_of(wl.torch_dtype)
    b, S, H, D, nc, r = wl.b, wl.sq, wl.h, wl.d, wl.n_c, wl.ratio

    # compressor: every row
    c64 = oracle.compress(f64(inp["x"]), f64(inp["z"]), r, wl.span)
    check_close("c", buf.c, c64, tol)
    c_or = torch.tensor(c64).to(wl.torch_dtype).double().numpy()   # the single cast to dtype
    kv = f64(inp["kv"])
    sink = f64(inp["sink"])

    must = [0, 1, r - 1, r, wl.window - 1, wl.window, S - 1, S - 2]
    if wl.kprime:
        must += [wl.kprime * r - 2, wl.kprime * r - 1, wl.kprime * r]
    rows = sample_rows(b, S, n_rows, seed, must)
    rb, rt = rows[:, 0], rows[:, 1]

    if wl.topk > 0 and wl.kprime > 0:
        qi = f64(inp["q_i"][rb, rt])
        w = f64(inp["w"][rb, rt])
        dense = oracle.index_scores(qi, f64(inp["k_i"]), w, r, rows)
        oidx, _ = oracle.topk(dense, r, wl.topk, rows)
        gidx = buf.idx[rb, rt].cpu().numpy()
        gsc = buf.score[rb, rt].cpu().numpy()
        exact = check_topk_rows(gidx, gsc, oidx, dense, rt, r, nc, wl.kprime, score_tol=tol)
        say(f"  top-k rows identical: {exact}/{len(rows)}")
    else:
        gidx = None

    # attention forward on every sampled row, with the GPU's own index rows
    q_rows = f64(inp["q"][rb, rt])
    o_ref, lse_ref = oracle.attn_fwd(q_rows, kv, c_or, gidx, sink, wl.scale, wl.window, r, rows)
    check_close("out", buf.out[rb, rt], o_ref, tol)
    check_close("lse", buf.lse[rb, rt], lse_ref, tol)

    # backward with dO nonzero on one row of every query block of every batch row
    qb = csa.csa_sparse_attn_bwd_query_block(dm, wl.topk > 0 or wl.ratio > 1)
    assert qb > 0
    rows_b = _block_rows(b, S, qb, seed, n_bwd_rows)
    say(f"  backward: query blocks of {qb}, {len(rows_b)} rows with nonzero dO")
    do_m = torch.zeros_like(inp["do"])
    bb, bt = torch.tensor(rows_b[:, 0]).cuda(), torch.tensor(rows_b[:, 1]).cuda()
    do_m[bb, bt] = inp["do"][bb, bt]
    inp_b = dict(inp)
    inp_b["do"] = do_m
    inp.pop("q_i", None)
    pipeline.backward(dm, inp_b, buf, wl.scale)
    torch.cuda.synchronize()
    idx_b = None if gidx is None else buf.idx[bb, bt].cpu().numpy()
    rdq, rdkv, rdc, rds = oracle.attn_bwd(f64(inp["q"][bb, bt]), kv, c_or, idx_b, sink, wl.scale,
                                          wl.window, r, rows_b, f64(inp["do"][bb, bt]))
    check_close("dq (sampled rows)", buf.dq[bb, bt], rdq, tol)
    other = torch.ones(b, S, dtype=torch.bool, device="cuda")
    other[bb, bt] = False
    assert torch.count_nonzero(buf.dq[other]) == 0
    check_close("dkv", buf.dkv, rdkv, tol)
    check_close("dc", buf.dc, rdc, tol)
    check_close("dsink", buf.dsink, rds, tol)
    rdx, rdz = oracle.compress_bwd(f64(inp["x"]), f64(inp["z"]), rdc, r, wl.span)
    check_close("dx", buf.dx, rdx, tol)
    check_close("dz", buf.dz, rdz, tol)
    del buf, inp, inp_b, do_m
    torch.cuda.empty_cache()


LOSS_WORKLOADS = [n for n in csa_synth.WORKLOAD_ORDER if csa_synth.WORKLOADS[n].topk > 0]
N_LOSS_ROWS = {"tiny_f32": 128, "csa4_s4096": 32, "csa4_d512_s8192": 16, "csa4_s65536_skew": 12}


@pytest.mark.parametrize("name", LOSS_WORKLOADS)
def test_workload_indexer_loss(gpu, name):
    """The indexer's training path at full size after a full forward pass.

    The loss is linear in dkl, so a dkl that is zero except on sampled rows
    makes every gradient (the sampled rows of dq_i and dw, all of dk_i) an
    oracle computation over those rows.  The sampled rows are fed the
    oracle's selection, scores and LSE (and every row the oracle's
    compressed rows), so both sides see the same inputs there."""
    import compressed_sparse_attention_softmax_amd as csa
    from compressed_sparse_attention_softmax_amd import pipeline
    from oracle import indexer_loss as il
    wl = csa_synth.WORKLOADS[name]
    seed = csa_synth.WORKLOAD_SEEDS[name]
    say(f"[workload loss] {name} seed={seed} b={wl.b} sq={wl.sq} h={wl.h} d={wl.d} K={wl.topk} {wl.dtype}")
    torch.cuda.empty_cache()
    inp = csa_synth.make_inputs(wl, seed, device="cuda", parts=("attn", "compress", "index"))
    dm = csa.dims_of(wl)
    buf = pipeline.allocate(dm, wl.torch_dtype, wl.z_channels)
    pipeline.forward(dm, inp, buf, wl.scale)
    b, S, H, D, nc, r, kp = wl.b, wl.sq, wl.h, wl.d, wl.n_c, wl.ratio, wl.kprime
    c_or = torch.tensor(oracle.compress(f64(inp["x"]), f64(inp["z"]), r, wl.span)).to(wl.torch_dtype)
    must = [0, 1, r - 1, r, kp * r - 1, kp * r, S - 1]
    rows = sample_rows(b, S, N_LOSS_ROWS[name], seed + 7, must)
    rb, rt = rows[:, 0], rows[:, 1]
    qi_rows, w_rows = f64(inp["q_i"][rb, rt]), f64(inp["w"][rb, rt])
    dense = oracle.index_scores(qi_rows, f64(inp["k_i"]), w_rows, r, rows)
    oidx, osc = oracle.topk(dense, r, wl.topk, rows)
    q_rows = f64(inp["q"][rb, rt])
    _, lse_rows = oracle.attn_fwd(q_rows, f64(inp["kv"]), f64(c_or), oidx, f64(inp["sink"]), wl.scale,
                                  wl.window, r, rows)
    bt = (torch.tensor(rb).cuda(), torch.tensor(rt).cuda())
    buf.idx[bt] = torch.tensor(oidx, dtype=torch.int32).cuda()
    score32 = torch.tensor(osc, dtype=torch.float32)
    buf.score[bt] = score32.cuda()
    lse32 = torch.tensor(lse_rows, dtype=torch.float32)
    buf.lse[bt] = lse32.cuda()
    gen = torch.Generator().manual_seed(seed + 9)
    dkl = torch.zeros(b, S, device="cuda")
    dkl_rows = torch.randn(len(rows), generator=gen)
    dkl[bt] = dkl_rows.cuda()
    lbuf = pipeline.allocate_loss(dm, wl.torch_dtype)
    pipeline.indexer_loss(dm, inp, buf, lbuf, wl.scale, dkl, c=c_or.cuda())
    torch.cuda.synchronize()
    tol = tol_of(wl.torch_dtype)
    target = il.teacher_target(q_rows, f64(c_or), f64(lse32), oidx, wl.scale, r, rows)
    r_kl, predict = il.kl_loss(target, f64(score32))
    check_close("kl (sampled rows)", lbuf.kl[bt], r_kl, tol)
    rdq, rdw, rdk, _ = il.loss_bwd(qi_rows, f64(inp["k_i"]), w_rows, oidx, r, rows, target, predict,
                                   dkl_rows.double().numpy())
    check_close("dq_i (sampled rows)", lbuf.dq_i[bt], rdq, tol)
    check_close("dw (sampled rows)", lbuf.dw[bt], rdw, tol)
    other = torch.ones(b, S, dtype=torch.bool, device="cuda")
    other[bt] = False
    assert torch.count_nonzero(lbuf.dq_i[other]) == 0 and torch.count_nonzero(lbuf.dw[other]) == 0
    check_close("dk_i", lbuf.dk_i, rdk, tol)
    del buf, lbuf, inp
    torch.cuda.empty_cache()


def test_workload_dsa_gqa(gpu):
    """The simplified DSA over GQA at its bench size (b1 sq4096 h32 h_kv8
    d128/128, K'=512): the GPU's one-head selection on sampled rows against
    the oracle's (near-tie band rule), then attention fed the oracle's
    selection for every row, checked on sampled rows, with dO zero except on
    those rows so that dk and dv are oracle computations over them."""
    import compressed_sparse_attention_softmax_amd as csa
    from oracle import dsa_gqa
    wl = csa_synth.GQA_WORKLOADS["dsa_gqa_s4096"]
    say(f"[workload dsa gqa] {wl}")
    inp = csa_synth.make_gqa_inputs(wl, 8, device="cuda")
    b, S, kp = wl.b, wl.sq, wl.kprime
    dm = csa.make_dims(b, S, ratio=1, idx_heads=1, idx_dim=wl.idx_dim, topk=wl.topk)
    gidx = torch.empty(b, S, kp, dtype=torch.int32, device="cuda")
    gsc = torch.empty(b, S, kp, device="cuda")
    csa.csa_index_topk(dm, inp["q_i"], inp["k_i"], None, gidx, gsc)
    oidx, _, _ = oracle.index_topk(f64(inp["q_i"]), f64(inp["k_i"]), np.ones((b, S, 1)), 1, wl.topk)
    oidx = np.asarray(oidx, dtype=np.int32).reshape(b, S, kp)
    rows = sample_rows(b, S, 24, 8, [0, 1, kp - 1, kp, S - 1])
    rb, rt = rows[:, 0], rows[:, 1]
    dense = oracle.index_scores(f64(inp["q_i"][rb, rt]), f64(inp["k_i"]), np.ones((len(rows), 1)), 1, rows)
    exact = check_topk_rows(gidx[rb, rt].cpu().numpy(), gsc[rb, rt].cpu().numpy(), oidx[rb, rt], dense, rt, 1, S, kp,
                            score_tol=tol_of(wl.torch_dtype))
    say(f"  top-k rows identical: {exact}/{len(rows)}")
    g = csa.csa_gqa_dims(b, S, wl.h, wl.h_kv, wl.d_qk, wl.d_v, wl.topk)
    dt = wl.torch_dtype
    out = torch.empty(b, S, wl.h, wl.d_v, dtype=dt, device="cuda")
    lse = torch.empty(b, S, wl.h, device="cuda")
    ws = torch.empty(csa.csa_dsa_gqa_workspace(g, dt, True), dtype=torch.uint8, device="cuda")
    idx_d = torch.tensor(oidx).cuda()
    csa.csa_dsa_gqa_fwd(g, inp["q"], inp["k"], inp["v"], idx_d, wl.scale, out, lse, ws)
    bt = (torch.tensor(rb).cuda(), torch.tensor(rt).cuda())
    do = torch.zeros_like(inp["do"])
    do[bt] = inp["do"][bt]
    dq = torch.empty_like(inp["q"])
    dk = torch.empty(b, S, wl.h_kv, wl.d_qk, device="cuda")
    dv = torch.empty(b, S, wl.h_kv, wl.d_v, device="cuda")
    csa.csa_dsa_gqa_bwd(g, inp["q"], inp["k"], inp["v"], idx_d, wl.scale, out, lse, do, dq, dk, dv, ws)
    torch.cuda.synchronize()
    q, k, v = (f64(inp[n]) for n in ("q", "k", "v"))
    ro, rl = dsa_gqa.fwd(q, k, v, oidx, wl.scale, rows=rows)
    tol = tol_of(dt)
    check_close("out (sampled rows)", out[bt], ro[rb, rt], tol)
    check_close("lse (sampled rows)", lse[bt], rl[rb, rt], tol)
    rdq, rdk, rdv = dsa_gqa.bwd(q, k, v, oidx, wl.scale, f64(out), f64(lse), f64(do), rows=rows)
    check_close("dq (sampled rows)", dq[bt], rdq[rb, rt], tol)
    other = torch.ones(b, S, dtype=torch.bool, device="cuda")
    other[bt] = False
    assert torch.count_nonzero(dq[other]) == 0
    check_close("dk", dk, rdk, tol)
    check_close("dv", dv, rdv, tol)
