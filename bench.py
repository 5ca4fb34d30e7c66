#!/usr/bin/env python3
"""Benchmark of the CSA hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input already resident in HBM:

    csa_compress -> csa_index_topk -> csa_sparse_attn_fwd
                 -> csa_sparse_attn_bwd -> csa_compress_bwd

all on the current HIP stream.  W untimed warm-up steps (continued until the
GPU has been busy SETTLE_S seconds, so that its clocks have settled), then
exactly K timed steps bracketed by device synchronisation, one HIP event pair
per step.  A second pass of K steps records per-stage events and times the
dominant kernel around each launch.

Prints one JSON line (metric, tokens/s, roofline of the dominant kernel, the
oracle's CPU baseline on a bounded sample).  ``--gpus N`` with N > 1 exits:
this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA fwd+bwd tokens/s + TFLOPS (% MFMA peak) at sq=4096, top-k=512, bf16"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0
STAGES = ["compress", "index_topk", "attn_fwd", "attn_bwd", "compress_bwd"]
# Continuous GPU work before the timed steps: the GPU raises its clocks over
# some tens of milliseconds of load (after an idle moment a step of the bench
# workload starts about 15 % slower and settles after about 50 steps), so the
# warm-up runs until the GPU has been busy this long.
SETTLE_S = 0.25


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def count_work(wl, idx):
    """Algorithmic work of one step: attention fwd = sum_{b,t} h * N_cand(t) * 2 * (d_qk + d_v),
    bwd = 2 x fwd, indexer = sum_{b,t} n_valid(t) * idx_heads * 2 * idx_dim.  Padding (-1)
    and not-yet-valid slots are never counted."""
    import torch
    dev = idx.device if idx is not None else "cpu"
    t = torch.arange(wl.sq, device=dev)
    nwin = torch.clamp(t + 1, max=wl.window)
    nv = torch.clamp((t + 1) // wl.ratio, max=wl.n_c)
    if idx is None:
        ncomp = nv.unsqueeze(0).expand(wl.b, -1)
    else:
        ncomp = ((idx >= 0) & (idx < nv.view(1, -1, 1))).sum(dim=2)
    n_cand = float((nwin.unsqueeze(0) + ncomp).sum().item())
    fwd = n_cand * wl.h * 2 * (2 * wl.d)
    indexer = float(nv.sum().item()) * wl.b * wl.idx_heads * 2 * wl.idx_dim if wl.topk > 0 else 0.0
    return dict(n_cand=n_cand, attn_fwd=fwd, attn_bwd=2 * fwd, indexer=indexer,
                avg_cand=n_cand / (wl.b * wl.sq))


def kernel_work(wl, work):
    """Algorithmic work of one launch of each kernel: (amount, unit, bound).

    The attention work splits by product: the forward kernel does Q.row and
    P.row; the dq kernel the dP and dQ products; the key-stationary kernel the
    dK and dV products (P^T dO and dS'^T Q).  Recomputed logits are not
    counted.  Memory-bound kernels count the bytes they must move."""
    e = 2 if wl.dtype == "bf16" else 4
    tok = wl.b * wl.sq
    nc_rows = wl.b * wl.n_c
    fl = work["attn_fwd"]
    return {
        "attn_query_fwd": (fl, "flop", "mfma"),
        "attn_query_dq": (fl, "flop", "mfma"),
        "attn_rows": (fl, "flop", "mfma"),
        "index_topk": (work["indexer"], "flop", "mfma"),
        "compress_fwd": (tok * (wl.d + wl.z_channels) * e + nc_rows * wl.d * e, "byte", "hbm"),
        "compress_bwd": (tok * (wl.d + wl.z_channels) * (e + 4) + nc_rows * wl.d * 4, "byte", "hbm"),
        "attn_reduce": ((tok + nc_rows) * wl.d * 4, "byte", "hbm"),
    }


def load_traffic(kernel, workload):
    """HBM traffic of `kernel` from the committed PMC summary, if it was taken
    on the current source of that kernel (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "compressed_sparse_attention_softmax_amd", "csrc", rec["source"])
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if digest != rec["source_sha256"]:
        return None
    return rec["traffic_bytes"]


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and the number of threads the
    oracle's OpenMP loops use."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return model, threads


def oracle_pass(wl, inp, rows, idx_rows=None):
    """One oracle pass over the listed query rows: compressor forward over the
    whole sequence, indexer scores + one full top-k, attention forward and
    backward for the rows, compressor backward.  Returns per-stage seconds.
    With idx_rows the attention uses that selection instead of the oracle's."""
    import numpy as np
    import torch
    import oracle

    def f(t):
        return t.detach().to("cpu", torch.float64).numpy()

    rb, rt = torch.tensor(rows[:, 0]), torch.tensor(rows[:, 1])
    x, z, kv = f(inp["x"]), f(inp["z"]), f(inp["kv"])
    q, do = f(inp["q"][rb, rt]), f(inp["do"][rb, rt])
    sink = f(inp["sink"])
    sec = {}
    t0 = time.perf_counter()
    c = oracle.compress(x, z, wl.ratio, wl.span)
    sec["compress"] = time.perf_counter() - t0
    idx = None
    if wl.topk > 0:
        t0 = time.perf_counter()
        dense = oracle.index_scores(f(inp["q_i"][rb, rt]), f(inp["k_i"]), f(inp["w"][rb, rt]), wl.ratio, rows)
        idx, _ = oracle.topk(dense, wl.ratio, wl.topk, rows)
        del dense
        sec["index_topk"] = time.perf_counter() - t0
    if idx_rows is not None:
        idx = idx_rows
    t0 = time.perf_counter()
    oracle.attn_fwd(q, kv, c, idx, sink, wl.scale, wl.window, wl.ratio, rows)
    sec["attn_fwd"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    _, _, dc, _ = oracle.attn_bwd(q, kv, c, idx, sink, wl.scale, wl.window, wl.ratio, rows, do)
    sec["attn_bwd"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.compress_bwd(x, z, dc, wl.ratio, wl.span)
    sec["compress_bwd"] = time.perf_counter() - t0
    return sec


def stratified_rows(wl, n):
    import numpy as np
    n = min(n, wl.b * wl.sq)
    tt = np.linspace(0, wl.sq - 1, max(1, n // wl.b)).round().astype(np.int64)
    return np.array([(bi, t) for bi in range(wl.b) for t in np.unique(tt)], dtype=np.int64)


def cpu_baseline(wl, inp, seed, target_rows):
    """The oracle (as it stands) on a bounded, stratified sample of query rows:
    indexer scores + top-k + attention fwd + bwd for those rows, plus the
    compressor fwd + bwd over the whole sequence scaled to the sample."""
    rows = stratified_rows(wl, target_rows)
    sec = oracle_pass(wl, inp, rows)
    frac = len(rows) / (wl.b * wl.sq)
    t_rows = sum(v for k, v in sec.items() if k not in ("compress", "compress_bwd"))
    t_comp = sec["compress"] + sec["compress_bwd"]
    t_total = t_rows + t_comp * frac
    model, threads = host_cpu()
    what = ("every query row (a full pass)" if len(rows) == wl.b * wl.sq
            else f"{len(rows)} query rows stratified over t")
    out = {"value": len(rows) / t_total, "unit": "tokens/s", "cores": threads, "cpu_model": model,
           "kind": "oracle",
           "sample": (f"{what} (indexer + top-k + attention fwd + bwd, {t_rows:.1f} s) plus compressor "
                      f"fwd+bwd over all rows ({t_comp:.1f} s) scaled by {frac:.4f}; fp64; every stage runs "
                      f"OpenMP loops on {threads} threads (the backward deals rows to 16 fixed chunks, summed "
                      f"in chunk order)")}
    rep = os.path.join(ROOT, "profiles", "cpu_oracle_passes.json")
    if os.path.exists(rep):
        rec = json.load(open(rep))
        out["per_config"] = {"from": "profiles/cpu_oracle_passes.json (full oracle passes measured on the "
                                     "GPU host by its command; not re-run by this line)",
                             "cpu_model": rec.get("cpu_model"), "threads": rec.get("threads"),
                             "configs": {k: {"tokens_per_s": v["tokens_per_s"], "seconds": v["seconds"],
                                             "extrapolated": v["extrapolated"]}
                                         for k, v in rec.get("configs", {}).items()}}
    return out


def cpu_oracle_report(max_rows, only=None):
    """Full oracle passes (every query row) of each workload whose b*sq is at
    most max_rows; larger ones run a stratified sample of max_rows rows whose
    row-dependent time is scaled to all rows (flagged as extrapolated).
    Prints one JSON object; progress goes to stderr."""
    import csa_synth
    model, threads = host_cpu()
    res = {"cpu_model": model, "threads": threads, "max_rows": max_rows, "configs": {}}
    for name in csa_synth.WORKLOAD_ORDER:
        if only and name not in only:
            continue
        wl = csa_synth.WORKLOADS[name]
        inp = csa_synth.make_inputs(wl, csa_synth.WORKLOAD_SEEDS[name], device="cpu")
        n_all = wl.b * wl.sq
        rows = stratified_rows(wl, min(n_all, max_rows))
        log(f"oracle pass {name}: {len(rows)} of {n_all} rows ...")
        sec = oracle_pass(wl, inp, rows)
        frac = len(rows) / n_all
        row_t = sum(v for k, v in sec.items() if k not in ("compress", "compress_bwd"))
        total = sec["compress"] + sec["compress_bwd"] + row_t / frac
        res["configs"][name] = {"rows": int(len(rows)), "rows_total": n_all, "extrapolated": frac < 1.0,
                                "seconds": total, "tokens_per_s": n_all / total,
                                "stage_seconds": {k: round(v, 3) for k, v in sec.items()}}
        log(f"oracle pass {name}: {total:.1f} s ({'extrapolated from ' + str(len(rows)) + ' rows' if frac < 1 else 'full'})")
        del inp
    print(json.dumps(res), flush=True)


def bench_compress_epilogue(wl, dm, inp, buf, stream, K):
    """The compressor with its epilogue (RMS norm and RoPE on 64 channels,
    base 40000), forward and backward, timed over K calls each with events
    on the step's stream (not part of the step).  The epilogue kernel's
    algorithmic bytes: forward, the cast rows read and written
    (2 * b * n_c * d * e); backward, x and z over every block's span, dc read
    and dy written (fp32)."""
    import torch
    import compressed_sparse_attention_softmax_amd as csa
    D = wl.d
    g = torch.Generator().manual_seed(3)
    epi = dict(norm_w=(1.0 + 0.1 * torch.randn(D, generator=g)).cuda(), norm_eps=1e-6, rope_dim=min(64, D),
               rope_base=40000.0)
    dnw = torch.empty(D, device="cuda")
    ws = torch.empty(max(csa.csa_compress_bwd_workspace(dm), 16), dtype=torch.uint8, device="cuda")
    fwd = lambda: csa.csa_compress(dm, inp["x"], inp["z"], buf.c, None, stream=stream, **epi)
    bwd = lambda: csa.csa_compress_bwd(dm, inp["x"], inp["z"], buf.dc, buf.dx, buf.dz, stream=stream,
                                       dnorm_w=dnw, ws=ws, **epi)
    out = {}
    for name, fn in (("fwd", fwd), ("bwd", bwd)):
        fn()
        csa.csa_timing_enable(csa.CSA_K_COMPRESS_EPI)
        fn()
        n, ms = csa.csa_timing_read()
        csa.csa_timing_enable(-1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[f"{name}_ms_per_call"] = e0.elapsed_time(e1) / K
        out[f"{name}_epilogue_kernel_ms"] = ms / max(n, 1)
    e = 2 if wl.dtype == "bf16" else 4
    rows = wl.b * wl.n_c
    span_rows = rows * min(wl.span, wl.sq)
    fb = 2 * rows * D * e
    bb = span_rows * (D + wl.z_channels) * e + rows * D * 8
    out["fwd_epilogue_gbs"] = fb / (out["fwd_epilogue_kernel_ms"] * 1e-3) / 1e9
    out["bwd_epilogue_gbs"] = bb / (out["bwd_epilogue_kernel_ms"] * 1e-3) / 1e9
    out["config"] = {"norm": "rms, learned weight", "rope_dim": epi["rope_dim"], "rope_base": 40000.0}
    # leave the step's buffers as the plain step made them
    csa.csa_compress(dm, inp["x"], inp["z"], buf.c, None, stream=stream)
    torch.cuda.synchronize()
    log(f"bench: compressor with epilogue: {out}")
    return out


def bench_dsa_gqa(stream, K):
    """The simplified DSA over GQA (its own synthetic workload, b1 sq4096 h32
    h_kv8 d128/128, K'=512, one-head indexer with d_i 128): indexer, attention
    forward and backward, each timed over K calls with events on the stream.
    Algorithmic work: indexer 2 * d_i per (query, key <= t); attention
    forward 2 * (d_qk + d_v) per (query, head, valid selected key), backward
    twice that (the packed zero halves are not counted)."""
    import torch
    import csa_synth
    import compressed_sparse_attention_softmax_amd as csa
    wl = csa_synth.GQA_WORKLOADS["dsa_gqa_s4096"]
    inp = csa_synth.make_gqa_inputs(wl, 8, device="cuda")
    b, S, kp = wl.b, wl.sq, wl.kprime
    dm = csa.make_dims(b, S, ratio=1, idx_heads=1, idx_dim=wl.idx_dim, topk=wl.topk)
    g = csa.csa_gqa_dims(b, S, wl.h, wl.h_kv, wl.d_qk, wl.d_v, wl.topk)
    idx = torch.empty(b, S, kp, dtype=torch.int32, device="cuda")
    out = torch.empty(b, S, wl.h, wl.d_v, dtype=wl.torch_dtype, device="cuda")
    lse = torch.empty(b, S, wl.h, device="cuda")
    dq = torch.empty_like(inp["q"])
    dk = torch.empty(b, S, wl.h_kv, wl.d_qk, device="cuda")
    dv = torch.empty(b, S, wl.h_kv, wl.d_v, device="cuda")
    ws = torch.empty(csa.csa_dsa_gqa_workspace(g, wl.torch_dtype, True), dtype=torch.uint8, device="cuda")
    calls = {
        "indexer": lambda: csa.csa_index_topk(dm, inp["q_i"], inp["k_i"], None, idx, None, stream=stream),
        "attn_fwd": lambda: csa.csa_dsa_gqa_fwd(g, inp["q"], inp["k"], inp["v"], idx, wl.scale, out, lse, ws,
                                                stream=stream),
        "attn_bwd": lambda: csa.csa_dsa_gqa_bwd(g, inp["q"], inp["k"], inp["v"], idx, wl.scale, out, lse, inp["do"],
                                                dq, dk, dv, ws, stream=stream),
    }
    for fn in calls.values():
        fn()
    torch.cuda.synchronize()
    ms = {}
    for name, fn in calls.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / K
    t = torch.arange(S, device="cuda").view(1, -1, 1)
    nsel = float(((idx >= 0) & (idx <= t)).sum().item())
    fwd = nsel * wl.h * 2.0 * (wl.d_qk + wl.d_v)
    ind = float(b * S * (S + 1) / 2) * 2.0 * wl.idx_dim
    tf = {"indexer": ind, "attn_fwd": fwd, "attn_bwd": 2 * fwd}
    res = {"workload": {k: getattr(wl, k) for k in ("b", "sq", "h", "h_kv", "d_qk", "d_v", "topk", "idx_dim",
                                                   "dtype")},
           "ms": ms, "tokens_per_s": b * S / (sum(ms.values()) * 1e-3),
           "tflops": {k: tf[k] / (ms[k] * 1e-3) / 1e12 for k in ms}, "selected_keys": nsel}
    log(f"bench: dsa over gqa: {res}")
    return res


DENSE_LOSS_BUDGET = 64 << 20


def bench_indexer_loss_dense(wl, dm, inp, buf, stream, K):
    """The dense warm-up form of the indexer loss (every valid block is the
    support) on the step's inputs, its workspace planned for a 64 MiB budget,
    timed over K calls with events on the same stream (the step's LSE stands
    in for the warm-up's dense one: the timing does not depend on its values).

    Algorithmic work per (query, valid block): the teacher's logits 2*h*d, the
    student's <q_i, k_i> 2*HI*DI, the dq_i product 2*HI*DI (query kernel) and
    the dk_i product 2*HI*DI (key-stationary kernel); recomputed products are
    not counted.
    """
    import torch
    import compressed_sparse_attention_softmax_amd as csa
    ws_bytes = csa.csa_indexer_loss_dense_workspace(dm, DENSE_LOSS_BUDGET)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    b, S, nc = wl.b, wl.sq, wl.n_c
    kl = torch.empty(b, S, device="cuda")
    dkl = torch.full((b, S), 1.0 / (b * S), device="cuda")
    dq_i = torch.empty(b, S, wl.idx_heads, wl.idx_dim, dtype=wl.torch_dtype, device="cuda")
    dw = torch.empty(b, S, wl.idx_heads, device="cuda")
    dk_i = torch.empty(b, nc, wl.idx_dim, device="cuda")

    def call():
        csa.csa_indexer_loss_dense(dm, inp["q"], buf.c, buf.lse, inp["q_i"], inp["k_i"], inp["w"], wl.scale, kl=kl,
                                   dkl=dkl, dq_i=dq_i, dw=dw, dk_i=dk_i, ws=ws, stream=stream)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    kms = {}
    for k in (csa.CSA_K_LOSS_QUERY, csa.CSA_K_LOSS_KEYS, csa.CSA_K_LOSS_REDUCE):
        csa.csa_timing_enable(k)
        call()
        n, ms = csa.csa_timing_read()
        if n:
            kms[csa.csa_kernel_name(k)] = ms          # summed over the call's query chunks
    csa.csa_timing_enable(-1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_call = e0.elapsed_time(e1) / K
    pairs = float(b * sum(min((t + 1) // wl.ratio, nc) for t in range(S)))
    hd = 2.0 * wl.idx_heads * wl.idx_dim
    work = {"loss_query": pairs * (2.0 * wl.h * wl.d + 2 * hd), "loss_keys": pairs * hd}
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    kern = {}
    for k, fl in work.items():
        if k in kms:
            tf = fl / (kms[k] * 1e-3) / 1e12
            kern[k] = {"ms_per_call": kms[k], "algorithmic_flop": fl, "tflops": tf, "frac": tf / peak}
    log(f"bench: dense warm-up indexer loss {ms_call:.3f} ms/call, workspace {ws_bytes} B "
        f"(budget {DENSE_LOSS_BUDGET}); kernels(ms) {kms}")
    return {"ms_per_call": ms_call, "valid_blocks": pairs, "workspace_bytes": ws_bytes,
            "budget_bytes": DENSE_LOSS_BUDGET, "kernel_ms": kms, "kernels": kern,
            "timing": "HIP events on the launch stream; per-kernel times from the library's timing hook"}


def bench_indexer_loss(wl, dm, inp, buf, stream, K):
    """The indexer's training path after the step's forward (not part of the
    step): csa_indexer_loss over the selected blocks, scores and LSE the last
    step produced, timed over K calls with events on the same stream.

    Algorithmic work per (query, valid selected block): the teacher's logits
    2*h*d, the student's recomputed <q_i, k_i> 2*HI*DI and the dq_i product
    2*HI*DI (query kernel); the dk_i product 2*HI*DI (key-stationary kernel).
    """
    import torch
    import compressed_sparse_attention_softmax_amd as csa
    from compressed_sparse_attention_softmax_amd import pipeline
    lbuf = pipeline.allocate_loss(dm, wl.torch_dtype)
    dkl = torch.full((wl.b, wl.sq), 1.0 / (wl.b * wl.sq), device="cuda")

    def call():
        pipeline.indexer_loss(dm, inp, buf, lbuf, wl.scale, dkl, stream=stream)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    kms = {}
    for k in (csa.CSA_K_LOSS_QUERY, csa.CSA_K_LOSS_KEYS, csa.CSA_K_LOSS_REDUCE):
        csa.csa_timing_enable(k)
        call()
        call()
        n, ms = csa.csa_timing_read()
        if n:
            kms[csa.csa_kernel_name(k)] = ms / n
    csa.csa_timing_enable(-1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_call = e0.elapsed_time(e1) / K
    t = torch.arange(wl.sq, device="cuda")
    nv = torch.clamp((t + 1) // wl.ratio, max=wl.n_c).view(1, -1, 1)
    nsel = float(((buf.idx >= 0) & (buf.idx < nv)).sum().item())
    hd = 2.0 * wl.idx_heads * wl.idx_dim
    work = {"loss_query": nsel * (2.0 * wl.h * wl.d + 2 * hd), "loss_keys": nsel * hd}
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    kern = {}
    for k, fl in work.items():
        if k in kms:
            tf = fl / (kms[k] * 1e-3) / 1e12
            kern[k] = {"avg_launch_ms": kms[k], "algorithmic_flop": fl, "tflops": tf, "frac": tf / peak}
    log(f"bench: indexer loss {ms_call:.3f} ms/call; kernels(ms) {kms}")
    return {"ms_per_call": ms_call, "selected_blocks": nsel, "kernel_ms": kms, "kernels": kern,
            "timing": "HIP events on the launch stream; per-kernel times from the library's timing hook"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="csa4_s4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step only (skip the indexer loss, compressor epilogue and DSA-over-GQA lines)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step as one HIP graph replay (reported beside the eager headline)")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows of the oracle's CPU sample (default: every row of the bench workload, a "
                         "full oracle pass of a few seconds on the GPU host; fewer rows are a stratified sample)")
    ap.add_argument("--cpu-oracle-report", type=int, default=0, metavar="MAX_ROWS",
                    help="time full oracle passes of every workload (sampled and extrapolated above MAX_ROWS "
                         "query rows) on the host CPU, print one JSON object and exit (no GPU used)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 3 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.cpu_oracle_report:
        cpu_oracle_report(args.cpu_oracle_report)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this hot path runs on one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) "
              "is not supported. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import csa_synth
    import compressed_sparse_attention_softmax_amd as csa
    from compressed_sparse_attention_softmax_amd import pipeline

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    csa.load()
    wl = csa_synth.WORKLOADS[args.workload]
    seed = csa_synth.WORKLOAD_SEEDS[args.workload]
    dm = csa.dims_of(wl)
    inp = csa_synth.make_inputs(wl, seed, device="cuda")
    buf = pipeline.allocate(dm, wl.torch_dtype, wl.z_channels)
    stream = torch.cuda.current_stream()
    scale = wl.scale
    sink = inp["sink"]

    cur = {"s": stream}      # launch stream of the calls (None = the current stream, e.g. a capture stream)

    def stage_calls():
        yield lambda: csa.csa_compress(dm, inp["x"], inp["z"], buf.c, None, stream=cur["s"])
        yield (lambda: csa.csa_index_topk(dm, inp["q_i"], inp["k_i"], inp["w"], buf.idx, buf.score,
                                          stream=cur["s"])) if buf.idx is not None else None
        yield lambda: csa.csa_sparse_attn_fwd(dm, inp["q"], inp["kv"], buf.c, buf.idx, sink, scale, buf.out,
                                              buf.lse, stream=cur["s"])
        yield lambda: csa.csa_sparse_attn_bwd(dm, inp["q"], inp["kv"], buf.c, buf.idx, sink, scale, buf.out,
                                              buf.lse, inp["do"], buf.dq, buf.dkv, buf.dc, buf.dsink,
                                              ws=buf.ws, stream=cur["s"])
        yield lambda: csa.csa_compress_bwd(dm, inp["x"], inp["z"], buf.dc, buf.dx, buf.dz, stream=cur["s"])

    calls = list(stage_calls())

    # memory contract of the indexer: nothing beyond its inputs and outputs
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    if calls[1] is not None:
        calls[1]()
    torch.cuda.synchronize()
    index_peak_delta = torch.cuda.max_memory_allocated() - base

    def one_step():
        for c in calls:
            if c is not None:
                c()

    # the work counts read the step's selection on the host (the GPU idles):
    # they come before the warm-up
    one_step()
    torch.cuda.synchronize()
    work = count_work(wl, buf.idx)
    kwork = kernel_work(wl, work)

    # warm-up: W steps, then more until the GPU has been busy SETTLE_S seconds
    t_w = time.perf_counter()
    for _ in range(args.warmup):
        one_step()
    settle = 0
    while True:
        torch.cuda.synchronize()
        if time.perf_counter() - t_w >= SETTLE_S:
            break
        for _ in range(8):
            one_step()
        settle += 8

    # per-kernel durations (HIP events around each launch, two steps per
    # kernel, outside the timed region): picks the dominant kernel
    kernel_ms = {}
    for k in range(7):
        csa.csa_timing_enable(k)
        one_step()
        one_step()
        n, ms = csa.csa_timing_read()
        if n:
            kernel_ms[csa.csa_kernel_name(k)] = ms / n
    csa.csa_timing_enable(-1)
    dom_k = max(kernel_ms, key=kernel_ms.get)
    dom_id = [csa.csa_kernel_name(k) for k in range(7)].index(dom_k)

    K = args.steps

    def timed(run):
        """K steps, one pair of HIP events per step on the stream, bracketed by
        device synchronisation; returns (sorted step ms, wall seconds)."""
        step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K):
            step_ev[k][0].record(stream)
            run()
            step_ev[k][1].record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in step_ev), time.perf_counter() - t0

    def median(v):
        return v[K // 2] if K % 2 else 0.5 * (v[K // 2 - 1] + v[K // 2])

    # the headline: eager launches.  With --graph the step is also captured as
    # one HIP graph (the entry points enqueue kernels only: no memset nodes, no
    # host synchronisation) and its replays are reported beside it (on this
    # stack a replay has measured slower than the eager launches)
    step_ms, elapsed = timed(one_step)
    graph_ms = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        cur["s"] = None
        with torch.cuda.stream(side):
            one_step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        cur["s"] = stream
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        graph_ms = median(timed(graph.replay)[0])
    ms_median = median(step_ms)

    # a second pass of K steps (not the headline): per-stage events, and the
    # dominant kernel timed around every launch by the library's hook
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(K)]
    csa.csa_timing_enable(dom_id)
    torch.cuda.synchronize()
    for k in range(K):
        e = ev[k]
        e[0].record(stream)
        for i, c in enumerate(calls):
            if c is not None:
                c()
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    csa.csa_timing_enable(-1)
    n_dom, ms_dom = csa.csa_timing_read()
    dom_ms = ms_dom / max(n_dom, 1)

    stage_ms = {s: sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(K)) / K for i, s in enumerate(STAGES)}
    ms_step = ms_median
    tokens = wl.b * wl.sq
    flops_step = work["attn_fwd"] + work["attn_bwd"] + work["indexer"]
    attn_s = (stage_ms["attn_fwd"] + stage_ms["attn_bwd"]) * 1e-3
    attn_tflops = (work["attn_fwd"] + work["attn_bwd"]) / attn_s / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    amount, unit, bound = kwork[dom_k]
    if unit == "flop":
        achieved, r_unit, r_peak = amount / (dom_ms * 1e-3) / 1e12, "TFLOP/s", peak
    else:
        achieved, r_unit, r_peak = amount / (dom_ms * 1e-3) / 1e9, "GB/s", PEAK_HBM_GBS
    roofline = {"bound": bound, "achieved": achieved, "peak": r_peak, "unit": r_unit, "frac": achieved / r_peak,
                "traffic": load_traffic(dom_k, wl.name), "kernel": dom_k, "launches": n_dom,
                "avg_launch_ms": dom_ms, "algorithmic_per_launch": amount,
                "timing": "HIP events recorded on the launch stream around every launch of the kernel "
                          "in a second pass of the same K steps (the headline pass records only step events)"}
    result = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": ms_step,
        "ms_per_step_timing": "median of per-step HIP event pairs on the stream over the K timed steps (eager "
                              "launches), after the W warm-up steps and settle_steps more (the GPU busy "
                              f"{SETTLE_S} s before the timed steps)",
        "ms_per_step_wall_mean": elapsed * 1e3 / K,
        "ms_per_step_min_max": [step_ms[0], step_ms[-1]],
        "ms_per_step_graph_median": graph_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded normals, shapes and scales of the workload)",
        "config": {"workload": wl.name, "b": wl.b, "sq": wl.sq, "h": wl.h, "d": wl.d, "ratio": wl.ratio,
                   "span": wl.span, "window": wl.window, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim,
                   "topk": wl.topk, "parallelism": "single GPU"},
        "tflops": flops_step / (ms_step * 1e-3) / 1e12,
        "attention_tflops": attn_tflops,
        "attention_frac_of_mfma_peak": attn_tflops / peak,
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "work": {k: v for k, v in work.items()},
        "kernel_ms": {k: round(v, 5) for k, v in kernel_ms.items()},
        "roofline": roofline,
        "memory": {"index_topk_workspace_bytes": csa.csa_index_topk_workspace(dm),
                   "index_topk_peak_alloc_delta_bytes": int(index_peak_delta),
                   "max_allocated_bytes": int(torch.cuda.max_memory_allocated())},
        "cpu_baseline": None,
    }
    if not args.no_extras:
        if wl.topk > 0:
            result["indexer_loss"] = bench_indexer_loss(wl, dm, inp, buf, stream, K)
        if wl.n_c > 0:
            result["indexer_loss_dense"] = bench_indexer_loss_dense(wl, dm, inp, buf, stream, K)
        result["compress_epilogue"] = bench_compress_epilogue(wl, dm, inp, buf, stream, K)
        result["dsa_gqa"] = bench_dsa_gqa(stream, K)
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on a CPU sample ...")
        result["cpu_baseline"] = cpu_baseline(wl, inp, seed, args.cpu_rows)
    log(f"bench: {wl.name}: {ms_step:.3f} ms/step, {result['value']:.0f} tokens/s, "
        f"{result['tflops']:.1f} TFLOP/s; stages(ms) {result['stage_ms']}; attention {attn_tflops:.1f} TFLOP/s "
        f"({100 * attn_tflops / peak:.1f}% of peak); kernels(ms) {result['kernel_ms']}; "
        f"roofline {dom_k}: {achieved:.1f} {r_unit} ({100 * roofline['frac']:.1f}% of peak)")
    print(json.dumps(result), flush=True)
    if args.copy_mib > 0:
        # a plain device copy of known size: its FETCH_SIZE / WRITE_SIZE under
        # rocprofv3 calibrate the HBM byte counters of the kernels above
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copied {args.copy_mib} MiB x3 for counter calibration")


if __name__ == "__main__":
    main()
