"""Writes tests/golden/oracle_tiny.npz from the oracle alone.

A regression fixture: a small fp32 CSA layer (S=64) run through every oracle
step.  Inputs come from csa_synth; expected values only from ``oracle``.
Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import csa_synth  # noqa: E402
import oracle  # noqa: E402

WL = csa_synth.WORKLOADS["tiny_f32"].replace(sq=64, h=2, d=16, window=8, idx_dim=8, topk=6, z_channels=16)
SEED = 77


def compute():
    inp = {k: (None if v is None else v.double().numpy()) for k, v in csa_synth.make_inputs(WL, SEED).items()}
    c = oracle.compress(inp["x"], inp["z"], WL.ratio, WL.span)
    idx, sc, _ = oracle.index_topk(inp["q_i"], inp["k_i"], inp["w"], WL.ratio, WL.topk)
    rows = oracle.all_rows(WL.b, WL.sq)
    q = inp["q"].reshape(-1, WL.h, WL.d)
    o, lse = oracle.attn_fwd(q, inp["kv"], c, idx, inp["sink"], WL.scale, WL.window, WL.ratio, rows)
    dq, dkv, dc, dsink = oracle.attn_bwd(q, inp["kv"], c, idx, inp["sink"], WL.scale, WL.window,
                                         WL.ratio, rows, inp["do"].reshape(-1, WL.h, WL.d))
    dx, dz = oracle.compress_bwd(inp["x"], inp["z"], dc, WL.ratio, WL.span)
    return dict(c=c, idx=idx, score=sc, o=o, lse=lse, dq=dq, dkv=dkv, dc=dc, dsink=dsink, dx=dx, dz=dz)


if __name__ == "__main__":
    out = compute()
    np.savez_compressed(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.npz"), **out)
    print("wrote", sorted(out))
