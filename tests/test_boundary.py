"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects bad arguments on the host with the documented codes (no GPU call
is made for any of these)."""

import ctypes
import os
import re

import pytest

from variable_length_gqa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vlgqa.h")

EINVAL, EUNSUP = _lib.VLGQA_EINVAL, _lib.VLGQA_EUNSUPPORTED
BF16, F32 = _lib.VLGQA_BF16, _lib.VLGQA_F32
A = 0x10000          # a fake, 16-byte-aligned "device" address (never dereferenced)
MIS = 0x10008        # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def err(lib):
    return lib.vlgqa_last_error().decode()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("varlen_attention_fwd", "flash_attention_fwd", "flash_attention_fwd_fp8",
              "varlen_attention_bwd", "flash_attention_bwd", "flash_attention_decode",
              "vlgqa_decode_workspace_floats", "flash_attention_bwd_fp8",
              "vlgqa_bwd_workspace_floats", "flash_attention_decode_noalloc", "vlgqa_last_error",
              "vlgqa_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) <= set(_lib.SIGNATURES)
    assert lib.vlgqa_version().decode().startswith("vlgqa")


def varlen(lib, **kw):
    a = dict(q=A, k=A, v=A, cq=A, ck=A, tq=940, tk=940, b=3, h=4, hkv=4, mq=512, mk=512, d=64,
             causal=0, dtype=F32, out=A, lse=A)
    a.update(kw)
    return lib.varlen_attention_fwd(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["tq"], a["tk"],
                                    a["b"], a["h"], a["hkv"], a["mq"], a["mk"], a["d"],
                                    a["causal"], a["dtype"], a["out"], a["lse"], None)


def dense(lib, **kw):
    a = dict(q=A, k=A, v=A, b=4, h=32, hkv=8, sq=8192, cap=16384, d=128, causal=1, w=4096,
             n=8192, dtype=BF16, out=A, lse=A)
    a.update(kw)
    return lib.flash_attention_fwd(a["q"], a["k"], a["v"], a["b"], a["h"], a["hkv"], a["sq"],
                                   a["cap"], a["d"], a["causal"], a["w"], a["n"], a["dtype"],
                                   a["out"], a["lse"], None)


def fp8(lib, **kw):
    a = dict(q=A, k=A, v=A, b=8, h=32, hkv=8, sq=4096, sk=4096, d=128, causal=1, qs=0.01,
             ks=0.01, vs=0.01, os=0.01, out=A, lse=A)
    a.update(kw)
    return lib.flash_attention_fwd_fp8(a["q"], a["k"], a["v"], a["b"], a["h"], a["hkv"], a["sq"],
                                       a["sk"], a["d"], a["causal"], a["qs"], a["ks"], a["vs"],
                                       a["os"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code,arg", [
    (dict(h=6, hkv=4), EINVAL, "num_heads"),
    (dict(h=0), EINVAL, "num_heads"),
    (dict(hkv=0), EINVAL, "num_kv_heads"),
    (dict(d=96), EUNSUP, "head_dim"),
    (dict(d=256), EUNSUP, "head_dim"),
    (dict(dtype=7), EUNSUP, "dtype"),
    (dict(tq=-1), EINVAL, "total_q"),
    (dict(b=-2), EINVAL, "batch_size"),
    (dict(mq=-1), EINVAL, "max_seqlen_q"),
    (dict(causal=2), EINVAL, "causal"),
    (dict(q=0), EINVAL, "q"),
    (dict(k=MIS), EINVAL, "k"),
    (dict(cq=0), EINVAL, "cu_seqlens_q"),
    (dict(ck=MIS), EINVAL, "cu_seqlens_k"),
    (dict(out=0), EINVAL, "out"),
    (dict(lse=MIS), EINVAL, "lse"),
    (dict(tq=1 << 31), EINVAL, "total_q"),
])
def test_varlen_rejects(lib, kw, code, arg):
    assert varlen(lib, **kw) == code
    assert err(lib).startswith(arg + ":"), err(lib)


def test_varlen_empty_problems_return_ok_without_pointers(lib):
    assert varlen(lib, b=0, q=0, k=0, v=0, cq=0, ck=0, out=0, lse=0) == _lib.VLGQA_OK
    assert varlen(lib, tq=0, q=0, k=0, v=0, cq=0, ck=0, out=0, lse=0) == _lib.VLGQA_OK
    assert varlen(lib, tq=0, mq=0, q=0, k=0, v=0, cq=0, ck=0, out=0, lse=0) == _lib.VLGQA_OK
    assert err(lib) == ""


@pytest.mark.parametrize("kw,arg", [
    (dict(mq=0), "max_seqlen_q"),            # tokens but no room for any
    (dict(mq=313), "max_seqlen_q"),          # 3 * 313 < 940: some sequence is longer
    (dict(mk=300), "max_seqlen_k"),
])
def test_varlen_rejects_max_seqlen_below_the_average(lib, kw, arg):
    assert varlen(lib, **kw) == EINVAL
    assert err(lib).startswith(arg + ":"), err(lib)
    if arg == "max_seqlen_q":
        assert varlen_bwd(lib, **kw) == EINVAL
        assert err(lib).startswith(arg + ":"), err(lib)


@pytest.mark.parametrize("kw,code,arg", [
    (dict(n=16385), EINVAL, "kv_seq_len"),
    (dict(w=-1), EINVAL, "window_size"),
    (dict(h=32, hkv=5), EINVAL, "num_heads"),
    (dict(d=32), EUNSUP, "head_dim"),
    (dict(sq=-5), EINVAL, "seqlen_q"),
    (dict(cap=-1), EINVAL, "kv_capacity"),
    (dict(b=-1), EINVAL, "batch"),
    (dict(v=0), EINVAL, "v"),
    (dict(q=MIS), EINVAL, "q"),
    (dict(dtype=-1), EUNSUP, "dtype"),
])
def test_dense_rejects(lib, kw, code, arg):
    assert dense(lib, **kw) == code
    assert err(lib).startswith(arg + ":"), err(lib)


def test_dense_empty_problems_return_ok(lib):
    assert dense(lib, b=0, q=0, k=0, v=0, out=0, lse=0) == _lib.VLGQA_OK
    assert dense(lib, sq=0, q=0, k=0, v=0, out=0, lse=0) == _lib.VLGQA_OK


@pytest.mark.parametrize("kw,arg", [
    (dict(qs=0.0), "q_scale"), (dict(ks=-1.0), "k_scale"), (dict(vs=float("nan")), "v_scale"),
    (dict(os=float("inf")), "o_scale"), (dict(qs=1e-30, ks=1e-30), "q_scale"),
    (dict(h=4, hkv=3), "num_heads"), (dict(sk=-1), "kv_capacity"),
])
def test_fp8_rejects(lib, kw, arg):
    assert fp8(lib, **kw) == EINVAL
    assert err(lib).startswith(arg + ":"), err(lib)


def test_fp8_unsupported_head_dim(lib):
    assert fp8(lib, d=80) == EUNSUP


def test_python_binding_raises_without_touching_gpu():
    import torch

    import variable_length_gqa_amd as vg

    q = torch.zeros(4, 2, 64)
    with pytest.raises(ValueError):
        vg.varlen_attention_fwd(q, q, q, torch.zeros(2, dtype=torch.int32),
                                torch.zeros(2, dtype=torch.int32), 1, 2, 2, 4, 4, 64, False)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


# --------------------------------------------------------------------------
# backward entry points
# --------------------------------------------------------------------------

def varlen_bwd(lib, **kw):
    a = dict(do=A, q=A, k=A, v=A, o=A, lse=A, cq=A, ck=A, tq=940, tk=940, b=3, h=4, hkv=2,
             mq=512, mk=512, d=128, causal=1, dtype=BF16, dq=A, dk=A, dv=A, ws=A)
    a.update(kw)
    return lib.varlen_attention_bwd(a["do"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"],
                                    a["ck"], a["tq"], a["tk"], a["b"], a["h"], a["hkv"], a["mq"],
                                    a["mk"], a["d"], a["causal"], a["dtype"], a["dq"], a["dk"],
                                    a["dv"], a["ws"], None)


def dense_bwd(lib, **kw):
    a = dict(do=A, q=A, k=A, v=A, o=A, lse=A, b=2, h=8, hkv=2, sq=300, sk=300, d=64, causal=1,
             w=0, dtype=BF16, dq=A, dk=A, dv=A, ws=A)
    a.update(kw)
    return lib.flash_attention_bwd(a["do"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["b"],
                                   a["h"], a["hkv"], a["sq"], a["sk"], a["d"], a["causal"],
                                   a["w"], a["dtype"], a["dq"], a["dk"], a["dv"], a["ws"], None)


@pytest.mark.parametrize("kw,code,arg", [
    (dict(dtype=F32), EUNSUP, "dtype"),
    (dict(dtype=9), EUNSUP, "dtype"),
    (dict(d=96), EUNSUP, "head_dim"),
    (dict(h=6, hkv=4), EINVAL, "num_heads"),
    (dict(tk=-1), EINVAL, "total_k"),
    (dict(mk=-1), EINVAL, "max_seqlen_k"),
    (dict(causal=3), EINVAL, "causal"),
    (dict(cq=0), EINVAL, "cu_seqlens_q"),
    (dict(k=MIS), EINVAL, "k"),
    (dict(dk=0), EINVAL, "dk"),
    (dict(dv=MIS), EINVAL, "dv"),
    (dict(do=0), EINVAL, "dout"),
    (dict(o=MIS), EINVAL, "out"),
    (dict(lse=0), EINVAL, "lse"),
    (dict(dq=MIS), EINVAL, "dq"),
    (dict(ws=0), EINVAL, "workspace"),
    (dict(ws=MIS), EINVAL, "workspace"),
])
def test_varlen_bwd_rejects(lib, kw, code, arg):
    assert varlen_bwd(lib, **kw) == code
    assert err(lib).startswith(arg + ":"), err(lib)


@pytest.mark.parametrize("kw,code,arg", [
    (dict(dtype=F32), EUNSUP, "dtype"),
    (dict(d=32), EUNSUP, "head_dim"),
    (dict(w=-1), EINVAL, "window_size"),
    (dict(sk=-1), EINVAL, "seqlen_k"),
    (dict(b=-1), EINVAL, "batch"),
    (dict(h=8, hkv=3), EINVAL, "num_heads"),
    (dict(v=0), EINVAL, "v"),
    (dict(q=MIS), EINVAL, "q"),
    (dict(ws=MIS), EINVAL, "workspace"),
])
def test_dense_bwd_rejects(lib, kw, code, arg):
    assert dense_bwd(lib, **kw) == code
    assert err(lib).startswith(arg + ":"), err(lib)


def test_bwd_empty_problems_return_ok_without_pointers(lib):
    none = dict(do=0, q=0, k=0, v=0, o=0, lse=0, cq=0, ck=0, dq=0, dk=0, dv=0, ws=0)
    assert varlen_bwd(lib, b=0, **none) == _lib.VLGQA_OK
    assert varlen_bwd(lib, tq=0, tk=0, **none) == _lib.VLGQA_OK
    none.pop("cq"), none.pop("ck")
    assert dense_bwd(lib, b=0, **none) == _lib.VLGQA_OK
    assert dense_bwd(lib, sq=0, sk=0, **none) == _lib.VLGQA_OK
    assert err(lib) == ""


# --------------------------------------------------------------------------
# packing entry points
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kw,code,arg", [
    (dict(b=-1), EINVAL, "batch_size"),
    (dict(s=-1), EINVAL, "max_seqlen"),
    (dict(rb=24), EINVAL, "row_bytes"),
    (dict(rb=0), EINVAL, "row_bytes"),
    (dict(t=-1), EINVAL, "total"),
    (dict(t=1 << 31), EINVAL, "total"),
    (dict(cu=0), EINVAL, "cu_seqlens"),
    (dict(pad=MIS), EINVAL, "padded"),
    (dict(pk=0), EINVAL, "packed"),
])
def test_pack_rejects(lib, kw, code, arg):
    a = dict(pad=A, cu=A, b=3, s=512, rb=256, t=940, pk=A)
    a.update(kw)
    assert lib.vlgqa_pack(a["pad"], a["cu"], a["b"], a["s"], a["rb"], a["t"], a["pk"], None) == code
    assert err(lib).startswith(arg + ":"), err(lib)


def test_unpack_and_cu_seqlens_reject(lib):
    assert lib.vlgqa_unpack(A, A, 3, 512, 100, A, None) == EINVAL
    assert err(lib).startswith("row_bytes:")
    assert lib.vlgqa_unpack(A, A, 3, 512, 256, MIS, None) == EINVAL
    assert err(lib).startswith("padded:")
    assert lib.vlgqa_cu_seqlens(A, -1, A, None) == EINVAL
    assert lib.vlgqa_cu_seqlens(0, 4, A, None) == EINVAL
    assert err(lib).startswith("lengths:")
    assert lib.vlgqa_cu_seqlens(A, 4, 0, None) == EINVAL
    # nothing to move: OK without pointers
    assert lib.vlgqa_pack(0, 0, 0, 512, 256, 0, 0, None) == _lib.VLGQA_OK
    assert lib.vlgqa_unpack(0, A, 3, 0, 256, 0, None) == _lib.VLGQA_OK


def decode(lib, **kw):
    a = dict(q=A, k=A, v=A, b=16, h=32, hkv=8, sq=1, cap=16384, d=128, causal=1, w=0, n=8192,
             dtype=BF16, out=A, lse=A, ws=A, wsf=1 << 40)
    a.update(kw)
    return lib.flash_attention_decode(a["q"], a["k"], a["v"], a["b"], a["h"], a["hkv"], a["sq"],
                                      a["cap"], a["d"], a["causal"], a["w"], a["n"], a["dtype"],
                                      a["out"], a["lse"], a["ws"], a["wsf"], None)


@pytest.mark.parametrize("kw,code,arg", [
    (dict(sq=9), EINVAL, "seqlen_q"),           # 9 * 4 query rows > 32
    (dict(h=64, hkv=1), EINVAL, "seqlen_q"),
    (dict(n=16385), EINVAL, "kv_seq_len"),
    (dict(w=-1), EINVAL, "window_size"),
    (dict(dtype=F32), EUNSUP, "dtype"),
    (dict(d=96), EUNSUP, "head_dim"),
    (dict(h=32, hkv=5), EINVAL, "num_heads"),
    (dict(wsf=100), EINVAL, "workspace_floats"),
    (dict(ws=0), EINVAL, "workspace"),
    (dict(ws=MIS), EINVAL, "workspace"),
    (dict(k=0), EINVAL, "k"),
    (dict(causal=3), EINVAL, "causal"),
])
def test_decode_rejects(lib, kw, code, arg):
    assert decode(lib, **kw) == code
    assert err(lib).startswith(arg + ":"), err(lib)


def test_decode_empty_problems_and_workspace_size(lib):
    assert decode(lib, b=0, q=0, k=0, v=0, out=0, lse=0, ws=0, wsf=0) == _lib.VLGQA_OK
    assert decode(lib, sq=0, q=0, k=0, v=0, out=0, lse=0, ws=0, wsf=0) == _lib.VLGQA_OK
    f = lib.vlgqa_decode_workspace_floats
    assert f(-1, 8, 128, 100) == -1
    # one partial of 32 rows x (D + 2) floats per (batch, kv head, key slice);
    # the size never decreases as the attended length grows
    sizes = [f(16, 8, 128, n) for n in range(0, 20000, 97)]
    assert all(s % (16 * 8 * 32 * 130) == 0 and s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    assert decode(lib, wsf=f(16, 8, 128, 8192) - 1) == EINVAL


def bwd8(lib, **kw):
    a = dict(do=A, q=A, k=A, v=A, o=A, lse=A, b=8, h=32, hkv=8, sq=4096, sk=4096, d=128,
             causal=1, qs=0.01, ks=0.01, vs=0.01, dos=0.01, os=0.01, dqs=0.01, dks=0.01,
             dvs=0.01, dq=A, dk=A, dv=A, ws=A, wsf=1 << 40)
    a.update(kw)
    return lib.flash_attention_bwd_fp8(a["do"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["b"],
                                       a["h"], a["hkv"], a["sq"], a["sk"], a["d"], a["causal"],
                                       a["qs"], a["ks"], a["vs"], a["dos"], a["os"], a["dqs"],
                                       a["dks"], a["dvs"], a["dq"], a["dk"], a["dv"], a["ws"],
                                       a["wsf"], None)


@pytest.mark.parametrize("kw,code,arg", [
    (dict(qs=0.0), EINVAL, "q_scale"), (dict(dos=-1.0), EINVAL, "do_scale"),
    (dict(os=float("nan")), EINVAL, "o_scale"), (dict(dqs=float("inf")), EINVAL, "dq_scale"),
    (dict(dks=0.0), EINVAL, "dk_scale"), (dict(dvs=-2.0), EINVAL, "dv_scale"),
    (dict(qs=1e-30, ks=1e-30), EINVAL, "q_scale"),
    (dict(d=96), EUNSUP, "head_dim"), (dict(h=32, hkv=5), EINVAL, "num_heads"),
    (dict(sq=-1), EINVAL, "seqlen_q"), (dict(causal=2), EINVAL, "causal"),
    (dict(wsf=1000), EINVAL, "workspace_floats"), (dict(ws=MIS), EINVAL, "workspace"),
    (dict(k=0), EINVAL, "k"), (dict(q=MIS), EINVAL, "q"), (dict(dout=0), EINVAL, "dout"),
])
def test_bwd_fp8_rejects(lib, kw, code, arg):
    if "dout" in kw:
        kw = dict(do=kw.pop("dout"))
    assert bwd8(lib, **kw) == code
    assert err(lib).startswith(arg + ":"), err(lib)


def test_bwd_workspace_sizes(lib):
    f = lib.vlgqa_bwd_workspace_floats
    assert f(-1, 1, 1, 1, 64, 0) == -1
    # row planes rounded up to 16 bytes, then 4 D floats per key and kv head
    assert f(3, 5, 1, 1, 64, 0) == 8 + 4 * 5 * 64
    assert f(4, 5, 2, 1, 64, 0) == 16 + 4 * 5 * 64
    # E4M3: plus bf16 copies of q and dout (rows x heads) and of k (keys x kv heads)
    assert f(4, 5, 2, 1, 64, 1) == 16 + 4 * 5 * 64 + 4 * 2 * 64 + 5 * 1 * 64 // 2
    assert bwd8(lib, b=0, q=0, k=0, v=0, o=0, lse=0, dq=0, dk=0, dv=0, ws=0, wsf=0) == \
        _lib.VLGQA_OK


def test_sequences_past_32bit_buffer_offsets_are_rejected(lib):
    # one sequence's rows must span less than 4 GiB (the kernels' buffer
    # descriptors use 32-bit byte offsets): 300000 tokens x 64 heads x 128 x 2 B
    assert varlen(lib, h=64, hkv=8, d=128, dtype=BF16, mq=300000, mk=512, tq=300000,
                  tk=940) == EINVAL
    assert err(lib).startswith("max_seqlen_q:"), err(lib)
    assert varlen(lib, h=64, hkv=64, d=128, dtype=BF16, mq=512, mk=300000, tq=940,
                  tk=300000) == EINVAL
    assert err(lib).startswith("max_seqlen_k:"), err(lib)
    assert dense(lib, b=1, sq=1 << 24, cap=1 << 24, n=1 << 24) == EINVAL
    assert err(lib).startswith("seqlen_q:"), err(lib)
    assert decode(lib, b=1, cap=1 << 24, n=1 << 24) == EINVAL
    assert err(lib).startswith("kv_seq_len:"), err(lib)
    assert bwd8(lib, b=1, sq=64, sk=1 << 24) == EINVAL
    assert err(lib).startswith("seqlen_k:"), err(lib)
    # the FP8 forward reads V as a 16-bit copy: 20M keys x 128 x 2 B pass the
    # 1-byte code check but not the copy's
    assert fp8(lib, b=1, sq=64, sk=20_000_000) == EINVAL
    assert err(lib).startswith("kv_seq_len:"), err(lib)


def test_noalloc_decode_rejects_on_the_host(lib):
    # beyond the 4194304-float static scratch: 2048 x 8 (batch, kv head)
    # pairs need 16384 * 32 * 130 floats; checked before any HIP call
    assert lib.flash_attention_decode_noalloc(A, A, A, 2048, 64, 8, 1, 8192, 128, 1, 0, 8192,
                                              BF16, A, A, None) == EINVAL
    assert err(lib).startswith("batch:"), err(lib)
    assert lib.flash_attention_decode_noalloc(A, A, A, 2, 64, 8, 8, 8192, 128, 1, 0, 8192,
                                              BF16, A, A, None) == EINVAL
    assert err(lib).startswith("seqlen_q:"), err(lib)
    assert lib.flash_attention_decode_noalloc(A, A, A, 2, 64, 8, 1, 8192, 128, 1, 0, 8192,
                                              F32, A, A, None) == EUNSUP
    assert lib.flash_attention_decode_noalloc(A, A, A, 0, 64, 8, 1, 8192, 128, 1, 0, 8192,
                                              BF16, 0, 0, None) == _lib.VLGQA_OK
