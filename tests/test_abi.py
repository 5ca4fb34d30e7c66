"""The C ABI boundary without a GPU: the library loads, exports every symbol
include/csa.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import compressed_sparse_attention_softmax_amd as csa
from compressed_sparse_attention_softmax_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


def _lib():
    if not os.path.exists(csa.LIB_PATH):
        pytest.skip("libcsa.so not built")
    return csa.load()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_exactly_the_bound_names():
    assert header_functions() == sorted(_abi.EXPORTS)


def test_library_exports_every_header_symbol():
    lib = _lib()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.csa_version() == 9


def test_dims_struct_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct csa_dims \{(.*?)\} csa_dims;", src, re.S).group(1)
    names = re.findall(r"([a-z_]+)[,;]", body.replace("int32_t", ""))
    assert names == [f[0] for f in _abi.csa_dims._fields_]
    assert ctypes.sizeof(_abi.csa_dims) == 40


def _d(**kw):
    base = dict(b=1, sq=64, h=4, d=64, ratio=4, span=4, window=8, idx_heads=2, idx_dim=32, topk=8)
    base.update(kw)
    return _abi.csa_dims(*[base[f[0]] for f in _abi.csa_dims._fields_])


P = ctypes.c_void_p(16)   # a non-NULL address that is never dereferenced (validation fails first)
N = None


@pytest.mark.parametrize("fn,args,code", [
    ("csa_compress", lambda: (None, 0, P, P, 64, N, ctypes.c_float(1e-6), 0, ctypes.c_float(40000.0), P, N, N), -1),
    ("csa_compress", lambda: (ctypes.byref(_d()), 7, P, P, 64, N, ctypes.c_float(1e-6), 0, ctypes.c_float(40000.0), P, N, N), -3),
    ("csa_compress", lambda: (ctypes.byref(_d(ratio=0)), 0, P, P, 64, N, ctypes.c_float(1e-6), 0, ctypes.c_float(40000.0), P, N, N), -1),
    ("csa_compress", lambda: (ctypes.byref(_d(d=96)), 0, P, P, 96, N, ctypes.c_float(1e-6), 0, ctypes.c_float(40000.0), P, N, N), -4),
    ("csa_compress", lambda: (ctypes.byref(_d()), 0, P, P, 5, N, ctypes.c_float(1e-6), 0, ctypes.c_float(40000.0), P, N, N), -2),
    ("csa_compress", lambda: (ctypes.byref(_d()), 0, N, P, 64, N, ctypes.c_float(1e-6), 0, ctypes.c_float(40000.0), P, N, N), -1),
    ("csa_compress_bwd", lambda: (ctypes.byref(_d(sq=0)), 0, P, P, 64, N, ctypes.c_float(1e-6), 0, ctypes.c_float(40000.0), P, P, P, N, N, 0, N), -1),
    ("csa_index_topk", lambda: (ctypes.byref(_d(topk=0)), 0, P, P, P, N, P, N, N, 0, N), -1),
    ("csa_index_topk", lambda: (ctypes.byref(_d(idx_dim=48)), 0, P, P, P, N, P, N, N, 0, N), -4),
    ("csa_index_topk", lambda: (ctypes.byref(_d(idx_heads=65)), 0, P, P, P, N, P, N, N, 0, N), -4),
    ("csa_index_topk", lambda: (ctypes.byref(_d(sq=65536, topk=4096)), 1, P, P, P, N, P, N, N, 0, N), -4),
    ("csa_index_topk", lambda: (ctypes.byref(_d()), 0, P, N, P, N, P, N, N, 0, N), -1),
    ("csa_sparse_attn_fwd", lambda: (ctypes.byref(_d(h=65)), 0, P, P, P, P, N, N, ctypes.c_float(1.0), P, P, N), -4),
    ("csa_sparse_attn_fwd", lambda: (ctypes.byref(_d(window=0)), 0, P, P, P, P, N, N, ctypes.c_float(1.0), P, P, N), -1),
    ("csa_sparse_attn_fwd", lambda: (ctypes.byref(_d()), 0, P, P, N, P, N, N, ctypes.c_float(1.0), P, P, N), -1),
    ("csa_sparse_attn_fwd", lambda: (ctypes.byref(_d()), 0, P, P, P, P, N, N, ctypes.c_float(float("nan")), P, P, N), -1),
    ("csa_sparse_attn_fwd", lambda: (ctypes.byref(_d(d=512)), 0, P, P, P, P, N, N, ctypes.c_float(1.0), P, P, N), -4),
    ("csa_sparse_attn_fwd", lambda: (ctypes.byref(_d()), 0, P, P, P, P, N, N, ctypes.c_float(1.0), N, P, N), -1),
])
def test_validation_errors(fn, args, code):
    lib = _lib()
    rc = getattr(lib, fn)(*args())
    assert rc == code, (fn, rc, lib.csa_last_error())
    assert lib.csa_last_error().decode().startswith(fn)


@pytest.mark.parametrize("eps,rope_dim,base,code", [(float("nan"), 0, 1.0, -1), (-1.0, 0, 1.0, -1),
                                                    (1e-6, 3, 1.0, -1), (1e-6, 66, 1.0, -1), (1e-6, 8, 0.0, -1),
                                                    (1e-6, 8, float("inf"), -1)])
def test_compress_epilogue_validation(eps, rope_dim, base, code):
    lib = _lib()
    rc = lib.csa_compress(ctypes.byref(_d()), 0, P, P, 64, P, ctypes.c_float(eps), rope_dim, ctypes.c_float(base),
                          P, N, N)
    assert rc == code, lib.csa_last_error()


def test_compress_bwd_epilogue_workspace():
    lib = _lib()
    d = _d()
    need = lib.csa_compress_bwd_workspace(ctypes.byref(d))
    assert need >= 4 * d.b * (d.sq // d.ratio) * d.d
    # with the epilogue on, a missing or short workspace is rejected before any launch
    args = (ctypes.byref(d), 0, P, P, 64, N, ctypes.c_float(1e-6), 8, ctypes.c_float(40000.0), P, P, P, N)
    assert lib.csa_compress_bwd(*args, N, 0, N) == -5
    assert lib.csa_compress_bwd(*args, P, need - 4, N) == -5
    # dnorm_w needs norm_w
    assert lib.csa_compress_bwd(ctypes.byref(d), 0, P, P, 64, N, ctypes.c_float(1e-6), 0, ctypes.c_float(1.0),
                                P, P, P, P, N, 0, N) == -1


def _bwd(dq, dkv, dc, dsink, sink=P, c=P):
    lib = _lib()
    return lib.csa_sparse_attn_bwd(ctypes.byref(_d()), 0, P, P, c, P, N, sink, ctypes.c_float(1.0), P, P, P,
                                   dq, dkv, dc, dsink, N, 0, N)


@pytest.mark.parametrize("missing", ["dq", "dkv", "dc"])
def test_gradient_gate_is_all_or_nothing(missing):
    args = dict(dq=P, dkv=P, dc=P)
    args[missing] = N
    rc = _bwd(args["dq"], args["dkv"], args["dc"], N)
    assert rc == -1
    assert missing in _lib().csa_last_error().decode()


def test_index_topk_without_blocks_is_a_noop():
    # sq < ratio: K' = min(topk, n_c) = 0, so k_i, idx and score are empty (NULL)
    lib = _lib()
    assert lib.csa_index_topk(ctypes.byref(_d(sq=3)), 0, P, N, P, N, N, N, N, 0, N) == 0
    assert lib.csa_index_topk(ctypes.byref(_d(sq=3)), 0, N, N, P, N, N, N, N, 0, N) == -1
    assert lib.csa_index_topk(ctypes.byref(_d(sq=4)), 0, P, N, P, N, N, N, N, 0, N) == -1


def test_gradient_gate_all_null_is_a_noop():
    assert _bwd(N, N, N, N) == 0


def test_dsink_requires_sink():
    assert _bwd(N, N, N, P, sink=N) == -1


def test_dc_requires_compressed_rows():
    assert _bwd(P, P, P, N, c=N) == -1


def test_workspace_queries():
    lib = _lib()
    assert lib.csa_index_topk_workspace(ctypes.byref(_d())) == 0
    d = _d()
    need = lib.csa_sparse_attn_bwd_workspace(ctypes.byref(d))
    # at least Delta (b*sq*h floats) plus one query block's partial rows
    assert need >= 4 * (d.b * d.sq * d.h + (d.window - 1 + 32) * d.d + d.sq // d.ratio * d.d)
    assert lib.csa_sparse_attn_bwd_workspace(None) == 0


def test_workspace_too_small_is_rejected():
    lib = _lib()
    d = _d()
    need = lib.csa_sparse_attn_bwd_workspace(ctypes.byref(d))
    rc = lib.csa_sparse_attn_bwd(ctypes.byref(d), 0, P, P, P, P, N, P, ctypes.c_float(1.0), P, P, P,
                                 P, P, P, N, P, need - 4, N)
    assert rc == -5, lib.csa_last_error()
    rc = lib.csa_sparse_attn_bwd(ctypes.byref(d), 0, P, P, P, P, N, P, ctypes.c_float(1.0), P, P, P,
                                 P, P, P, N, N, 0, N)
    assert rc == -5


def _loss(dims=None, dkl=N, kl=P, dq_i=N, dw=N, dk_i=N, ws=N, ws_bytes=0, q_i=P, scale=1.0):
    lib = _lib()
    return lib.csa_indexer_loss(ctypes.byref(dims or _d()), 0, P, P, P, q_i, P, P, P, P, ctypes.c_float(scale),
                                dkl, kl, dq_i, dw, dk_i, ws, ws_bytes, N)


@pytest.mark.parametrize("kw,code", [
    (dict(dims=_d(idx_dim=48)), -4),
    (dict(dims=_d(idx_heads=65)), -4),
    (dict(dims=_d(h=65)), -4),
    (dict(dims=_d(d=96)), -4),
    (dict(dims=_d(topk=0)), -1),
    (dict(dims=_d(sq=65536, topk=4096)), -4),
    (dict(scale=float("inf")), -1),
    (dict(dkl=P), -1),                              # gradient gate: dq_i, dw, dk_i missing
    (dict(dkl=P, dq_i=P, dw=P), -1),
    (dict(dq_i=P, dw=P, dk_i=P), -1),               # gradients without dkl
    (dict(dkl=P, dq_i=P, dw=P, dk_i=P, q_i=N), -1),  # q_i required with gradients
    (dict(dkl=P, dq_i=P, dw=P, dk_i=P), -5),        # no workspace
])
def test_indexer_loss_validation(kw, code):
    rc = _loss(**kw)
    assert rc == code, (kw, rc, _lib().csa_last_error())
    assert _lib().csa_last_error().decode().startswith("csa_indexer_loss")


def test_indexer_loss_nothing_requested_is_a_noop_and_workspace():
    lib = _lib()
    assert _loss(kl=N) == 0
    d = _d()
    need = lib.csa_indexer_loss_workspace(ctypes.byref(d))
    kp = min(d.topk, d.sq // d.ratio)
    assert need >= 4 * (d.b * d.sq * kp + d.sq // d.ratio * d.idx_dim)
    assert _loss(dkl=P, dq_i=P, dw=P, dk_i=P, ws=P, ws_bytes=need - 4) == -5
    assert lib.csa_indexer_loss_workspace(None) == 0


def _g(**kw):
    base = dict(b=1, sq=64, h=8, h_kv=2, d_qk=64, d_v=64, topk=16)
    base.update(kw)
    return _abi.csa_gqa_dims(*[base[f[0]] for f in _abi.csa_gqa_dims._fields_])


@pytest.mark.parametrize("g,dtype,code", [
    (dict(h=7), 1, -2), (dict(h=256, h_kv=2), 1, -4), (dict(d_qk=128, d_v=64), 1, -4),
    (dict(d_qk=128, d_v=128), 0, -4), (dict(topk=0), 1, -1), (dict(sq=4096, topk=4096), 1, -4),
    (dict(d_qk=60, d_v=68), 1, -4), (dict(), 5, -3),
])
def test_dsa_gqa_validation(g, dtype, code):
    lib = _lib()
    rc = lib.csa_dsa_gqa_fwd(ctypes.byref(_g(**g)), dtype, P, P, P, P, ctypes.c_float(1.0), P, P, P, 1 << 30, N)
    assert rc == code, lib.csa_last_error()


def test_dsa_gqa_workspace_and_gate():
    lib = _lib()
    g = _g()
    need_f = lib.csa_dsa_gqa_workspace(ctypes.byref(g), 1, 0)
    need_b = lib.csa_dsa_gqa_workspace(ctypes.byref(g), 1, 1)
    assert 0 < need_f < need_b
    assert lib.csa_dsa_gqa_fwd(ctypes.byref(g), 1, P, P, P, P, ctypes.c_float(1.0), P, P, P, need_f - 1, N) == -5
    assert lib.csa_dsa_gqa_bwd(ctypes.byref(g), 1, P, P, P, P, ctypes.c_float(1.0), P, P, P, P, N, P, P,
                               need_b, N) == -1
    assert lib.csa_dsa_gqa_workspace(None, 1, 0) == 0


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="libcsa.so not found"):
        _abi.load(str(tmp_path / "missing.so"))


def test_timing_hook_without_launches():
    # host-only paths: enabling, reading with nothing recorded, names, bad ids
    lib = _lib()
    assert lib.csa_timing_enable(11) == -1
    assert lib.csa_timing_enable(-2) == -1
    assert lib.csa_timing_enable(csa.CSA_K_ATTN_ROWS) == 0
    assert csa.csa_timing_read() == (0, 0.0)
    assert lib.csa_timing_enable(-1) == 0
    names = [csa.csa_kernel_name(k) for k in range(11)]
    assert names == ["compress_fwd", "compress_bwd", "index_topk", "attn_query_fwd", "attn_query_dq",
                     "attn_rows", "attn_reduce", "loss_query", "loss_keys", "loss_reduce", "compress_epilogue"]
    assert csa.csa_kernel_name(99) == ""


M = ctypes.c_void_p(24)   # non-NULL and not 16-byte aligned (never dereferenced)
F1, F4 = ctypes.c_float(1.0), ctypes.c_float(40000.0)


def _fwd_args(**over):
    a = dict(q=P, kv=P, c=P, idx=P, doc=N, sink=P, out=P, lse=P)
    a.update(over)
    return (ctypes.byref(_d()), 1, a["q"], a["kv"], a["c"], a["idx"], a["doc"], a["sink"], F1, a["out"], a["lse"], N)


@pytest.mark.parametrize("name", ["q", "kv", "c", "idx", "sink", "out", "lse", "doc"])
def test_attn_fwd_rejects_misaligned_tensors(name):
    lib = _lib()
    rc = lib.csa_sparse_attn_fwd(*_fwd_args(**{name: M}))
    msg = lib.csa_last_error().decode()
    assert rc == -1 and "16-byte aligned" in msg and msg.split(": ")[1].startswith(name if name != "doc" else "doc_ids")


@pytest.mark.parametrize("pos,name", [(2, "q"), (3, "kv"), (4, "c"), (11, "dout"), (12, "dq"), (13, "dkv"),
                                      (14, "dc"), (15, "dsink")])
def test_attn_bwd_rejects_misaligned_tensors(pos, name):
    lib = _lib()
    args = [ctypes.byref(_d()), 1, P, P, P, P, N, P, F1, P, P, P, P, P, P, P, N, 0, N]
    args[pos] = M
    rc = lib.csa_sparse_attn_bwd(*args)
    assert rc == -1 and f"{name} is not 16-byte aligned" in lib.csa_last_error().decode()


@pytest.mark.parametrize("pos,name", [(2, "x"), (3, "z"), (9, "c"), (10, "c32")])
def test_compress_rejects_misaligned_tensors(pos, name):
    lib = _lib()
    args = [ctypes.byref(_d()), 1, P, P, 64, N, ctypes.c_float(1e-6), 0, F4, P, P, N]
    args[pos] = M
    rc = lib.csa_compress(*args)
    assert rc == -1 and f"{name} is not 16-byte aligned" in lib.csa_last_error().decode()


@pytest.mark.parametrize("pos,name", [(2, "x"), (3, "z"), (9, "dc"), (10, "dx"), (11, "dz")])
def test_compress_bwd_rejects_misaligned_tensors(pos, name):
    lib = _lib()
    args = [ctypes.byref(_d()), 1, P, P, 64, N, ctypes.c_float(1e-6), 0, F4, P, P, P, N, N, 0, N]
    args[pos] = M
    rc = lib.csa_compress_bwd(*args)
    assert rc == -1 and f"{name} is not 16-byte aligned" in lib.csa_last_error().decode()


@pytest.mark.parametrize("pos,name", [(2, "q_i"), (3, "k_i"), (4, "w"), (6, "idx"), (7, "score")])
def test_index_topk_rejects_misaligned_tensors(pos, name):
    lib = _lib()
    args = [ctypes.byref(_d()), 1, P, P, P, N, P, P, N, 0, N]
    args[pos] = M
    rc = lib.csa_index_topk(*args)
    assert rc == -1 and f"{name} is not 16-byte aligned" in lib.csa_last_error().decode()


def test_indexer_loss_rejects_misaligned_tensors():
    lib = _lib()
    rc = lib.csa_indexer_loss(ctypes.byref(_d()), 1, M, P, P, P, P, P, P, P, F1, N, P, N, N, N, N, 0, N)
    assert rc == -1 and "q is not 16-byte aligned" in lib.csa_last_error().decode()


def _sbhd(b=2, sq=64, h=4, d=64):
    """Element strides of sequence-major q [sq, b, h, d], kv [sq, b, d], lse [sq, b, h]."""
    return _abi.csa_attn_strides(h * d, b * h * d, d, d, b * d, h, b * h)


def _strided_fwd(st, dims=None, **over):
    a = dict(q=P, kv=P, c=P, idx=P, doc=N, sink=P, out=P, lse=P)
    a.update(over)
    return (ctypes.byref(dims or _d(b=2)), None if st is None else ctypes.byref(st), 1, a["q"], a["kv"], a["c"],
            a["idx"], a["doc"], a["sink"], F1, a["out"], a["lse"], N)


def test_strides_struct_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct csa_attn_strides \{(.*?)\} csa_attn_strides;", src, re.S).group(1)
    names = re.findall(r"([a-z_]+)[,;]", body.replace("int64_t", ""))
    assert names == [f[0] for f in _abi.csa_attn_strides._fields_]
    assert ctypes.sizeof(_abi.csa_attn_strides) == 56


@pytest.mark.parametrize("st", [None, "sbhd", "contiguous"])
def test_strided_fwd_accepts_valid_strides(st):
    # valid strides pass validation; the misaligned q is then what is reported
    lib = _lib()
    s = {"sbhd": _sbhd(), "contiguous": _abi.csa_attn_strides(64 * 4 * 64, 4 * 64, 64, 64 * 64, 64, 64 * 4, 4),
         None: None}[st]
    rc = lib.csa_sparse_attn_fwd_strided(*_strided_fwd(s, q=M))
    assert rc == -1 and "q is not 16-byte aligned" in lib.csa_last_error().decode()


@pytest.mark.parametrize("field,value,text", [
    ("q_s", 516, "stride q_s"),          # not a multiple of 8 bf16 elements
    ("kv_b", 0, "stride kv_b"),
    ("q_h", 32, "q strides"),            # heads overlap rows of 64
    ("kv_s", 32, "kv strides"),
    ("q_b", 512, "q strides"),           # batch and sequence alias
    ("lse_s", 1, "lse strides"),         # sequence steps inside the 4 heads
])
def test_strided_fwd_rejects_bad_strides(field, value, text):
    lib = _lib()
    st = _sbhd()
    setattr(st, field, value)
    rc = lib.csa_sparse_attn_fwd_strided(*_strided_fwd(st))
    assert rc == -1 and text in lib.csa_last_error().decode()


def test_strided_axes_of_extent_one_are_ignored():
    lib = _lib()
    st = _sbhd(b=1)
    st.q_b = st.kv_b = st.lse_b = 0          # b == 1: never multiplied by anything but 0
    rc = lib.csa_sparse_attn_fwd_strided(*_strided_fwd(st, dims=_d(b=1), q=M))
    assert rc == -1 and "q is not 16-byte aligned" in lib.csa_last_error().decode()


def test_strided_bwd_validates_strides_then_workspace():
    lib = _lib()
    args = [ctypes.byref(_d(b=2)), ctypes.byref(_sbhd()), 1, P, P, P, P, N, P, F1, P, P, P, P, P, P, P, N, 0, N]
    assert lib.csa_sparse_attn_bwd_strided(*args) == -5
    bad = _sbhd()
    bad.kv_s = 36
    args[1] = ctypes.byref(bad)
    assert lib.csa_sparse_attn_bwd_strided(*args) == -1
    assert "stride kv_s" in lib.csa_last_error().decode()


def test_strided_binding_checks_stride_agreement():
    # CPU tensors are refused before any stride logic runs; the stride helper
    # itself is checked on CPU views
    import torch
    q = torch.zeros(64, 2, 4, 64, dtype=torch.bfloat16).transpose(0, 1)
    kv = torch.zeros(64, 2, 64, dtype=torch.bfloat16).transpose(0, 1)
    lse = torch.zeros(64, 2, 4).transpose(0, 1)
    st = _abi.attn_strides_of(q, kv, lse)
    assert (st.q_b, st.q_s, st.q_h, st.kv_b, st.kv_s, st.lse_b, st.lse_s) == (256, 512, 64, 64, 128, 4, 8)
    with pytest.raises(ValueError, match="GPU tensor"):
        _abi._strided_ptr(q, (2, 64, 4, 64), torch.bfloat16, "q")


def _seq_major_compress(b=2, sq=64, d=64, zc=64):
    """Element strides of sequence-major x [sq, b, d] and z [sq, b, zc]."""
    return _abi.csa_compress_strides(d, b * d, zc, b * zc)


def _compress_strided(st, dims=None, x=P, z=P, zc=64):
    return (ctypes.byref(dims or _d(b=2)), None if st is None else ctypes.byref(st), 1, x, z, zc, N,
            ctypes.c_float(1e-6), 0, F4, P, N, N)


@pytest.mark.parametrize("name,cls,fields,size", [
    ("csa_compress_strides", "csa_compress_strides", ("x_b", "x_s", "z_b", "z_s"), 32),
    ("csa_index_strides", "csa_index_strides", ("qi_b", "qi_s", "qi_h", "ki_b", "ki_s", "w_b", "w_s"), 56),
])
def test_compress_and_index_stride_structs_match_header(name, cls, fields, size):
    src = open(HEADER).read()
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), src, re.S).group(1)
    names = re.findall(r"([a-z_]+)[,;]", body.replace("int64_t", ""))
    assert names == [f[0] for f in getattr(_abi, cls)._fields_] == list(fields)
    assert ctypes.sizeof(getattr(_abi, cls)) == size


@pytest.mark.parametrize("st", [None, "seq", "contiguous"])
def test_compress_strided_accepts_valid_strides(st):
    # valid strides pass validation; the misaligned x is then what is reported
    lib = _lib()
    s = {"seq": _seq_major_compress(), "contiguous": _abi.csa_compress_strides(64 * 64, 64, 64 * 64, 64), None: None}[st]
    rc = lib.csa_compress_strided(*_compress_strided(s, x=M))
    assert rc == -1 and "x is not 16-byte aligned" in lib.csa_last_error().decode()


@pytest.mark.parametrize("field,value,text", [
    ("x_s", 132, "stride x_s"),          # not a multiple of 8 bf16 elements
    ("z_b", 0, "stride z_b"),
    ("x_s", 32, "x strides"),            # tokens overlap rows of 64 channels
    ("z_b", 64 * 2, "z strides"),        # batch and sequence alias
])
def test_compress_strided_rejects_bad_strides(field, value, text):
    lib = _lib()
    st = _seq_major_compress()
    setattr(st, field, value)
    rc = lib.csa_compress_strided(*_compress_strided(st))
    assert rc == -1 and text in lib.csa_last_error().decode()


def test_compress_strided_scalar_gate_strides_need_no_alignment():
    # z_channels = 1: the gate is read one element at a time
    lib = _lib()
    st = _abi.csa_compress_strides(64, 2 * 64, 1, 2)
    rc = lib.csa_compress_strided(*_compress_strided(st, x=M, zc=1))
    assert rc == -1 and "x is not 16-byte aligned" in lib.csa_last_error().decode()


def test_compress_bwd_strided_validates_strides():
    lib = _lib()
    st = _seq_major_compress()
    st.x_s = 36
    rc = lib.csa_compress_bwd_strided(ctypes.byref(_d(b=2)), ctypes.byref(st), 1, P, P, 64, N, ctypes.c_float(1e-6),
                                      0, F4, P, P, P, N, N, 0, N)
    assert rc == -1 and "stride x_s" in lib.csa_last_error().decode()


def _seq_major_index(b=2, sq=64, hi=2, di=32, nc=16):
    """Element strides of sequence-major q_i [sq, b, hi, di], k_i [nc, b, di], w [sq, b, hi]."""
    return _abi.csa_index_strides(hi * di, b * hi * di, di, di, b * di, hi, b * hi)


@pytest.mark.parametrize("field,value,text", [
    ("qi_s", 68, "stride qi_s"),         # not a multiple of 8 bf16 elements
    ("qi_h", 16, "q_i strides"),         # heads overlap rows of 32
    ("ki_s", 16, "k_i strides"),
    ("w_s", 1, "w strides"),             # tokens step inside the 2 heads
    ("w_b", 0, "stride w_b"),
])
def test_index_topk_strided_rejects_bad_strides(field, value, text):
    lib = _lib()
    st = _seq_major_index()
    setattr(st, field, value)
    rc = lib.csa_index_topk_strided(ctypes.byref(_d(b=2)), ctypes.byref(st), 1, P, P, P, N, P, P, N, 0, N)
    assert rc == -1 and text in lib.csa_last_error().decode()


def test_index_topk_strided_accepts_valid_strides():
    lib = _lib()
    rc = lib.csa_index_topk_strided(ctypes.byref(_d(b=2)), ctypes.byref(_seq_major_index()), 1, M, P, P, N, P, P, N,
                                    0, N)
    assert rc == -1 and "q_i is not 16-byte aligned" in lib.csa_last_error().decode()


def test_index_topk_strided_ignores_w_strides_without_w():
    # w == NULL (unit weights): its strides are never used and not checked
    lib = _lib()
    st = _seq_major_index()
    st.w_b = st.w_s = 0
    rc = lib.csa_index_topk_strided(ctypes.byref(_d(b=2)), ctypes.byref(st), 1, M, P, N, N, P, P, N, 0, N)
    assert rc == -1 and "q_i is not 16-byte aligned" in lib.csa_last_error().decode()


def test_compress_and_index_stride_helpers():
    import torch
    x = torch.zeros(64, 2, 64, dtype=torch.bfloat16).transpose(0, 1)
    z = torch.zeros(64, 2, 1, dtype=torch.bfloat16).transpose(0, 1)
    st = _abi.compress_strides_of(x, z)
    assert (st.x_b, st.x_s, st.z_b, st.z_s) == (64, 128, 1, 2)
    q_i = torch.zeros(64, 2, 2, 32, dtype=torch.bfloat16).transpose(0, 1)
    k_i = torch.zeros(16, 2, 32, dtype=torch.bfloat16).transpose(0, 1)
    w = torch.zeros(64, 2, 2).transpose(0, 1)
    si = _abi.index_strides_of(q_i, k_i, w)
    assert (si.qi_b, si.qi_s, si.qi_h, si.ki_b, si.ki_s, si.w_b, si.w_s) == (64, 128, 32, 32, 64, 2, 4)


def _dense_args(dims, **over):
    a = dict(q=P, c=P, lse=P, q_i=P, k_i=P, w=P, dkl=N, kl=P, dq_i=N, dw=N, dk_i=N, ws=N, ws_bytes=0)
    a.update(over)
    return (ctypes.byref(dims), 1, a["q"], a["c"], a["lse"], a["q_i"], a["k_i"], a["w"], F1, a["dkl"], a["kl"],
            a["dq_i"], a["dw"], a["dk_i"], a["ws"], a["ws_bytes"], N)


def test_dense_loss_workspace_plan_follows_the_budget():
    lib = _lib()
    dm = _d(b=1, sq=4096, h=64, d=128, ratio=4, idx_heads=64, idx_dim=128, topk=512)
    nc = 4096 // 4
    least = lib.csa_indexer_loss_dense_workspace(ctypes.byref(dm), 0)
    full = lib.csa_indexer_loss_dense_workspace(ctypes.byref(dm), 1 << 40)
    assert 0 < least < full
    assert least >= 2 * nc * 4                 # at least one query's two rows
    assert full >= 2 * 4096 * nc * 4           # every query's rows at once
    prev = least
    for budget in (least, least + 1, 3 * least, 10 << 20, 50 << 20, full - 1, full, 2 * full):
        got = lib.csa_indexer_loss_dense_workspace(ctypes.byref(dm), budget)
        assert got <= max(budget, least) and got >= prev
        prev = got
    assert lib.csa_indexer_loss_dense_workspace(ctypes.byref(dm), 2 * full) == full
    # topk plays no part in the dense form
    dm2 = _d(b=1, sq=4096, h=64, d=128, ratio=4, idx_heads=64, idx_dim=128, topk=0)
    assert lib.csa_indexer_loss_dense_workspace(ctypes.byref(dm2), 10 << 20) == \
        lib.csa_indexer_loss_dense_workspace(ctypes.byref(dm), 10 << 20)
    assert lib.csa_indexer_loss_dense_workspace(None, 0) == 0


def test_dense_loss_validation():
    lib = _lib()
    dm = _d(topk=0)
    need = lib.csa_indexer_loss_dense_workspace(ctypes.byref(dm), 0)
    # nothing requested: a no-op, no workspace needed
    assert lib.csa_indexer_loss_dense(*_dense_args(dm, kl=N)) == 0
    # kl alone still needs the workspace rows
    assert lib.csa_indexer_loss_dense(*_dense_args(dm)) == -5
    assert lib.csa_indexer_loss_dense(*_dense_args(dm, ws=P, ws_bytes=need - 1)) == -5
    assert "at least" in lib.csa_last_error().decode()
    # gradient gate
    assert lib.csa_indexer_loss_dense(*_dense_args(dm, dkl=P, dq_i=P, ws=P, ws_bytes=need)) == -1
    assert "gradient gate" in lib.csa_last_error().decode()
    # inputs of the student are required
    assert lib.csa_indexer_loss_dense(*_dense_args(dm, q_i=N, ws=P, ws_bytes=need)) == -1
    assert lib.csa_indexer_loss_dense(*_dense_args(dm, q=M, ws=P, ws_bytes=need)) == -1
    assert "q is not 16-byte aligned" in lib.csa_last_error().decode()
    assert lib.csa_indexer_loss_dense(*_dense_args(dm, ws=M, ws_bytes=need)) == -1
    assert lib.csa_indexer_loss_dense(*_dense_args(_d(idx_dim=48), ws=P, ws_bytes=need)) == -4
    assert lib.csa_indexer_loss_dense(*_dense_args(dm, ws=P, ws_bytes=need)[:1] + (7,) +
                                      _dense_args(dm, ws=P, ws_bytes=need)[2:]) == -3
