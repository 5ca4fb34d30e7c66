"""The whole pass captured in a HIP graph and replayed: every entry point
enqueues kernels only (no memset nodes, no host synchronisation), and the
reductions run in a fixed order, so each replay must reproduce the eager
results bit for bit, with other eager work on the stream between replays."""
import pytest
import torch

import csa_synth

pytestmark = pytest.mark.gpu


def test_pass_replays_bit_identical_in_a_graph(gpu):
    import compressed_sparse_attention_softmax_amd as csa
    from compressed_sparse_attention_softmax_amd import pipeline
    from parity import say
    wl = csa_synth.WORKLOADS["csa4_s4096"].replace(sq=520, topk=64)
    say(f"[graph] sq={wl.sq} K={wl.topk}")
    inp = csa_synth.make_inputs(wl, 5, device="cuda")
    dm = csa.dims_of(wl)
    ref = pipeline.allocate(dm, wl.torch_dtype, wl.z_channels)
    pipeline.step(dm, inp, ref, wl.scale)
    torch.cuda.synchronize()
    buf = pipeline.allocate(dm, wl.torch_dtype, wl.z_channels)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pipeline.step(dm, inp, buf, wl.scale)             # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pipeline.step(dm, inp, buf, wl.scale)
    names = ["c", "idx", "score", "out", "lse", "dq", "dkv", "dc", "dsink", "dx", "dz"]
    for rep in range(3):
        for n in names:                                     # scribble between replays
            t = getattr(buf, n)
            t.fill_(7 if t.dtype == torch.int32 else 7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            a, b = getattr(buf, n), getattr(ref, n)
            assert torch.equal(a, b), f"replay {rep}: {n} differs from the eager pass"
    say("  three replays identical to the eager pass")
