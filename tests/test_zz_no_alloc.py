"""The allocation-free backward (csa_sparse_attn_bwd_noalloc), called through
the C ABI, against csa_sparse_attn_bwd with a caller workspace: two calls in a
row, the second with a smaller input, each checked element by element (both
run the same kernels in the same fixed order, so they agree bit for bit; the
bar of the float tolerance is stated anyway).  The scratch keeps the first
call's contents when the second runs."""
import pytest
import torch

import csa_synth

pytestmark = pytest.mark.gpu


def _case(wl, seed):
    import compressed_sparse_attention_softmax_amd as csa
    from compressed_sparse_attention_softmax_amd import pipeline
    inp = csa_synth.make_inputs(wl, seed, device="cuda")
    dm = csa.dims_of(wl)
    ref = pipeline.allocate(dm, wl.torch_dtype, wl.z_channels)
    pipeline.forward(dm, inp, ref, wl.scale)
    pipeline.backward(dm, inp, ref, wl.scale)
    dq = torch.full_like(ref.dq, 7.0)
    dkv = torch.full_like(ref.dkv, 7.0)
    dc = torch.full_like(ref.dc, 7.0)
    dsink = torch.full_like(ref.dsink, 7.0)
    csa.csa_sparse_attn_bwd_noalloc(dm, inp["q"], inp["kv"], ref.c, ref.idx, inp["sink"], wl.scale, ref.out,
                                    ref.lse, inp["do"], dq, dkv, dc, dsink)
    torch.cuda.synchronize()
    for name, got, want in (("dq", dq, ref.dq), ("dkv", dkv, ref.dkv), ("dc", dc, ref.dc),
                            ("dsink", dsink, ref.dsink)):
        assert torch.equal(got, want), name
        tol = 1e-2 if wl.torch_dtype == torch.bfloat16 else 1e-5
        err = (got.float() - want.float()).abs().max().item()
        assert err <= tol * want.float().abs().max().item(), name


def test_noalloc_backward_matches_workspace_backward_twice(gpu):
    base = csa_synth.WORKLOADS["csa4_s4096"]
    _case(base, 31)                                        # the bench shape (44.5 MiB of scratch)
    _case(base.replace(sq=1500, topk=200), 32)             # then a smaller one on the same scratch


def test_noalloc_backward_rejects_dims_beyond_the_scratch(gpu):
    import compressed_sparse_attention_softmax_amd as csa
    wl = csa_synth.WORKLOADS["csa4_d512_s8192"]             # needs 564 MiB of scratch
    dm = csa.dims_of(wl)
    assert csa.csa_sparse_attn_bwd_workspace(dm) > 64 << 20
    lib = csa.load()
    import ctypes
    P = ctypes.c_void_p(256)
    rc = lib.csa_sparse_attn_bwd_noalloc(ctypes.byref(dm), 1, P, P, P, P, None, P, ctypes.c_float(0.05), P, P, P,
                                         P, P, P, P, None)
    assert rc == -4 and "scratch" in lib.csa_last_error().decode()
