"""Host logic of bench.py, without a GPU: the one-GPU guard, the algorithmic
work it divides by (counted from the index rows, padding never counted), and
the HBM-traffic lookup that is only trusted for the kernel source the
counters were taken on."""
import json
import os
import subprocess
import sys

import torch

import bench
import csa_synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and not r.stdout.strip()


def _hand_count(wl, idx):
    """Candidates of every (b, t): window rows min(t + 1, W) plus the valid
    entries of the index row (0 <= j < (t+1) // ratio), by plain loops."""
    n = 0
    for bi in range(wl.b):
        for t in range(wl.sq):
            nv = min((t + 1) // wl.ratio, wl.n_c)
            win = min(t + 1, wl.window)
            if idx is None:
                comp = nv
            else:
                comp = sum(1 for j in idx[bi, t].tolist() if 0 <= j < nv)
            n += win + comp
    return n


def test_work_counts_valid_candidates_only():
    wl = csa_synth.WORKLOADS["tiny_f32"].replace(b=2, sq=37)
    g = torch.Generator().manual_seed(3)
    # index rows with padding, entries not yet valid and a duplicate
    idx = torch.randint(-1, wl.n_c + 3, (wl.b, wl.sq, wl.kprime), generator=g, dtype=torch.int32)
    idx[:, :, 1] = idx[:, :, 0]
    w = bench.count_work(wl, idx)
    n = _hand_count(wl, idx)
    assert w["n_cand"] == n
    assert w["attn_fwd"] == n * wl.h * 2 * (2 * wl.d)
    assert w["attn_bwd"] == 2 * w["attn_fwd"]
    nv_sum = sum(min((t + 1) // wl.ratio, wl.n_c) for t in range(wl.sq))
    assert w["indexer"] == wl.b * nv_sum * wl.idx_heads * 2 * wl.idx_dim


def test_work_dense_mode_and_window_only_rows():
    wl = csa_synth.WORKLOADS["hca128_s16384"].replace(sq=300)
    w = bench.count_work(wl, None)
    assert w["n_cand"] == _hand_count(wl, None)
    assert w["indexer"] == 0.0                      # no indexer on the dense layer
    empty = torch.full((1, 40, 4), -1, dtype=torch.int32)
    wl2 = csa_synth.WORKLOADS["tiny_f32"].replace(sq=40, topk=4)
    assert bench.count_work(wl2, empty)["n_cand"] == sum(min(t + 1, wl2.window) for t in range(40))


def test_kernel_work_splits_the_attention_products():
    wl = csa_synth.WORKLOADS["csa4_s4096"]
    work = dict(attn_fwd=1e9, attn_bwd=2e9, indexer=5e8)
    k = bench.kernel_work(wl, work)
    # three kernels, two of the six products each; their sum is fwd + bwd
    assert k["attn_query_fwd"][0] + k["attn_query_dq"][0] + k["attn_rows"][0] == work["attn_fwd"] + work["attn_bwd"]
    assert k["index_topk"][0] == work["indexer"]
    assert k["compress_fwd"][2] == "hbm" and k["attn_rows"][2] == "mfma"


def test_traffic_is_trusted_only_for_the_profiled_source(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_attn_rows_csa4_s4096.json")))
    got = bench.load_traffic("attn_rows", "csa4_s4096")
    assert got is None or got == rec["traffic_bytes"]
    # the same record against a source with another hash is not trusted
    fake_root = tmp_path
    (fake_root / "profiles").mkdir()
    src_dir = fake_root / "compressed_sparse_attention_softmax_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (src_dir / rec["source"]).write_text("// a different kernel source\n")
    (fake_root / "profiles" / "traffic_attn_rows_csa4_s4096.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    assert bench.load_traffic("attn_rows", "csa4_s4096") is None
    assert bench.load_traffic("attn_rows", "no_such_workload") is None
