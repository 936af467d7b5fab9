"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status codes
before making any HIP call (only invalid calls are made here)."""
import ctypes
import os
import re

import pytest

import exact_attention_46_amd as ea
from exact_attention_46_amd import build as ea_build

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "mi355attn.h")

A = ctypes.c_void_p(4096)   # aligned, non-NULL stand-ins: never dereferenced,
A2 = ctypes.c_void_p(8192)  # every call below fails validation first
MIS = ctypes.c_void_p(4098)
A16 = ctypes.c_void_p(4096 + 16)  # 16-byte but not 256-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:long\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text,
                      flags=re.M)


def header_defines():
    out = {}
    for name, val in re.findall(r"#define\s+(MI355ATTN_\w+)\s+\(?(-?\d+)\)?", open(HEADER).read()):
        out[name] = int(val)
    return out


@pytest.fixture(scope="module")
def lib():
    return ea.load_library()


def test_library_built_for_gfx950():
    assert ea_build.ARCH == "gfx950"
    assert os.path.exists(ea.LIB_PATH)


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert sorted(names) == sorted(ea.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_codes_match_header(lib):
    d = header_defines()
    assert d["MI355ATTN_OK"] == ea._binding.OK
    assert d["MI355ATTN_ERR_NULL_PTR"] == ea._binding.ERR_NULL_PTR
    assert d["MI355ATTN_ERR_BAD_SHAPE"] == ea._binding.ERR_BAD_SHAPE
    assert d["MI355ATTN_ERR_UNSUPPORTED"] == ea._binding.ERR_UNSUPPORTED
    assert d["MI355ATTN_ERR_MISALIGNED"] == ea._binding.ERR_MISALIGNED
    assert d["MI355ATTN_ERR_BAD_ARG"] == ea._binding.ERR_BAD_ARG
    assert d["MI355ATTN_ERR_HIP"] == ea._binding.ERR_HIP
    assert d["MI355ATTN_ERR_SCRATCH"] == ea._binding.ERR_SCRATCH
    assert d["MI355ATTN_BF16"] == 0 and d["MI355ATTN_FP16"] == 1
    for code in range(-6, 1):
        s = ea.attn_status_str(code)
        assert s and s != "unknown status"
    assert ea.attn_status_str(123) == "unknown status"


def fwd(lib, q=A, k=A, v=A, o=A2, lse=A2, B=1, Hq=2, Hkv=2, Nq=8, Nk=8, d=128, scale=0.1,
        causal=1, dtype=0):
    return lib.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(lse=None), -1),
    (dict(B=0), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(Nq=0), -2), (dict(Nk=-1), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(B=2**30, Hq=2**10, Nq=128 * 4), -2),
    (dict(Nq=2**23 + 1), -2), (dict(Nk=2**23 + 1), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(dtype=2), -3),
    (dict(scale=0.0), -5), (dict(scale=-1.0), -5), (dict(scale=float("nan")), -5),
    (dict(scale=float("inf")), -5), (dict(causal=2), -5),
    (dict(q=MIS), -4), (dict(o=MIS), -4), (dict(lse=ctypes.c_void_p(4097)), -4),
])
def test_attn_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def bwd(lib, q=A, k=A, v=A, o=A, do=A, lse=A2, delta=A2, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=2,
        Nq=8, Nk=8, d=128, scale=0.1, causal=1, dtype=0):
    return lib.attn_bwd(q, k, v, o, do, lse, delta, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                        causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(do=None), -1), (dict(lse=None), -1),
    (dict(delta=None), -1), (dict(dq=None), -1), (dict(dk=None), -1), (dict(dv=None), -1),
    (dict(B=0), -2), (dict(Hkv=0), -2), (dict(Nq=0), -2), (dict(Nk=-3), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(Nq=2**23 + 1), -2),
    (dict(B=2**20, Hq=2**10, Hkv=2**10, Nq=128 * 4), -2),
    (dict(d=32), -3), (dict(dtype=5), -3),
    (dict(scale=0.0), -5), (dict(scale=float("nan")), -5), (dict(causal=-1), -5),
    (dict(do=MIS), -4), (dict(dk=MIS), -4), (dict(delta=ctypes.c_void_p(4099)), -4),
])
def test_attn_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def bwd_noalloc(lib, q=A, k=A, v=A, o=A, do=A, lse=A2, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=2,
                Nq=8, Nk=8, d=128, scale=0.1, causal=1, dtype=0):
    return lib.attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                                causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(dv=None), -1),
    (dict(B=0), -2), (dict(Hq=3, Hkv=2), -2), (dict(Nq=2**23 + 1), -2),
    (dict(d=32), -3), (dict(dtype=5), -3),
    (dict(scale=0.0), -5), (dict(causal=2), -5), (dict(do=MIS), -4),
    # one D per query row: at most 2^22 rows fit the fixed scratch
    (dict(B=1, Hq=33, Hkv=1, Nq=2**17), -7), (dict(B=2, Hq=32, Hkv=8, Nq=2**16 + 1), -7),
])
def test_attn_bwd_noalloc_rejects(lib, kw, code):
    assert bwd_noalloc(lib, **kw) == code


def bwd_ds(lib, q=A, k=A, v=A, o=A, do=A, lse=A2, delta=A2, ds=A, ds_bytes=1 << 20, dq=A,
           dk=A, dv=A, B=1, Hq=2, Hkv=2, Nq=8, Nk=8, d=128, scale=0.1, causal=1, dtype=0):
    return lib.attn_bwd_ds(q, k, v, o, do, lse, delta, ds, ds_bytes, dq, dk, dv, B, Hq, Hkv, Nq,
                           Nk, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(delta=None), -1), (dict(ds=None), -1),
    (dict(B=0), -2), (dict(Hq=3, Hkv=2), -2), (dict(Nk=2**23 + 1), -2),
    (dict(d=32), -3), (dict(dtype=4), -3),
    (dict(scale=float("nan")), -5), (dict(causal=-1), -5),
    (dict(ds=A16), -4), (dict(delta=MIS), -4),
    # the workspace must hold B * Hq * ceil(Nk / 64) * ceil(Nq / 128) blocks of 16 KiB
    (dict(ds_bytes=2 * 16384 - 1), -5), (dict(ds_bytes=0), -5),
])
def test_attn_bwd_ds_rejects(lib, kw, code):
    assert bwd_ds(lib, **kw) == code


def test_attn_bwd_ds_workspace_sizes(lib):
    # B * Hq * ceil(Nk / 64) * ceil(Nq / 128) blocks of 64 x 128 values of 2 bytes
    n = lib.attn_bwd_ds_workspace(1, 2, 8, 8)
    assert n == 2 * 16384
    assert lib.attn_bwd_ds_workspace(4, 32, 2048, 2048) == 4 * 32 * 2048 * 2048 * 2
    assert lib.attn_bwd_ds_workspace(1, 1, 129, 65) == 2 * 2 * 16384
    assert lib.attn_bwd_ds_workspace(0, 1, 1, 1) == -2
    assert lib.attn_bwd_ds_workspace(1, 1, 2**23 + 1, 1) == -2


def fwd_varlen(lib, q=A, k=A, v=A, o=A2, lse=A2, cq=A, ck=A2, B=3, Hq=4, Hkv=2, total_q=100,
               total_k=120, max_q=60, d=128, scale=0.1, causal=1, dtype=0):
    return lib.attn_fwd_varlen(q, k, v, o, lse, cq, ck, B, Hq, Hkv, total_q, total_k, max_q, d,
                               scale, causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(cq=None), -1), (dict(ck=None), -1),
    (dict(B=0), -2), (dict(total_q=0), -2), (dict(total_k=0), -2), (dict(max_q=0), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(max_q=2**23 + 1), -2), (dict(B=2**20, Hq=2**8, max_q=2**16), -2),
    (dict(d=96), -3), (dict(dtype=9), -3),
    (dict(scale=-2.0), -5), (dict(causal=3), -5),
    (dict(v=MIS), -4), (dict(cq=ctypes.c_void_p(4098)), -4),
])
def test_attn_fwd_varlen_rejects(lib, kw, code):
    assert fwd_varlen(lib, **kw) == code


def fwd_local(lib, q=A, k=A, v=A, o=A2, lse=A2, B=1, Hq=2, Hkv=2, Nq=8, Nk=8, d=128, scale=0.1,
              wl=4, wr=0, dtype=0):
    return lib.attn_fwd_local(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, wl, wr, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(B=0), -2), (dict(Nk=0), -2),
    (dict(Hq=3, Hkv=2), -2), (dict(Nq=2**23 + 1), -2), (dict(d=48), -3), (dict(dtype=3), -3),
    (dict(scale=float("nan")), -5), (dict(k=MIS), -4),
])
def test_attn_fwd_local_rejects(lib, kw, code):
    assert fwd_local(lib, **kw) == code


def qkvp(lib, qkv=A, o=A2, lse=A2, B=2, N=64, H=4, d=128, scale=0.1, causal=1, dtype=0):
    return lib.attn_fwd_qkvpacked(qkv, o, lse, B, N, H, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(qkv=None), -1), (dict(o=None), -1), (dict(lse=None), -1), (dict(B=0), -2), (dict(N=0), -2),
    (dict(H=0), -2), (dict(N=2**23 + 1), -2), (dict(d=32), -3), (dict(dtype=4), -3),
    (dict(scale=-1.0), -5), (dict(causal=7), -5), (dict(qkv=MIS), -4),
])
def test_attn_fwd_qkvpacked_rejects(lib, kw, code):
    assert qkvp(lib, **kw) == code


def split(lib, q=A, kc=A, vc=A, sl=A2, po=A2, pl=A2, B=2, Hq=8, Hkv=2, max_len=64, d=128,
          chunk=16, scale=0.1, dtype=0):
    return lib.attn_decode_split(q, kc, vc, sl, po, pl, B, Hq, Hkv, max_len, d, chunk, scale,
                                 dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kc=None), -1), (dict(sl=None), -1), (dict(po=None), -1),
    (dict(B=0), -2), (dict(max_len=0), -2), (dict(chunk=0), -2), (dict(Hq=6, Hkv=4), -2),
    (dict(d=80), -3), (dict(dtype=5), -3), (dict(Hq=66, Hkv=2), -3),
    (dict(scale=0.0), -5), (dict(kc=MIS), -4), (dict(sl=ctypes.c_void_p(4098)), -4),
    (dict(B=2**20, Hkv=2**10, max_len=2**20, chunk=1), -2), (dict(max_len=2**23 + 1), -2),
])
def test_attn_decode_split_rejects(lib, kw, code):
    assert split(lib, **kw) == code


def split_paged(lib, q=A, kp=A, vp=A, bt=A2, sl=A2, po=A2, pl=A2, B=2, Hq=8, Hkv=2,
                num_pages=10, page_size=32, max_pages=4, d=128, chunk=64, scale=0.1, dtype=0):
    return lib.attn_decode_split_paged(q, kp, vp, bt, sl, po, pl, B, Hq, Hkv, num_pages,
                                       page_size, max_pages, d, chunk, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kp=None), -1), (dict(bt=None), -1), (dict(pl=None), -1),
    (dict(B=0), -2), (dict(num_pages=0), -2), (dict(page_size=0), -2), (dict(max_pages=0), -2),
    (dict(chunk=0), -2), (dict(Hq=6, Hkv=4), -2), (dict(max_pages=2**18, page_size=64), -2),
    (dict(d=80), -3), (dict(dtype=7), -3), (dict(Hq=66, Hkv=2), -3),
    (dict(page_size=24), -3), (dict(chunk=40), -3), (dict(page_size=16, chunk=512), -3),
    (dict(page_size=48, chunk=800), -3),
    (dict(scale=float("nan")), -5), (dict(vp=MIS), -4), (dict(bt=ctypes.c_void_p(4098)), -4),
])
def test_attn_decode_split_paged_rejects(lib, kw, code):
    assert split_paged(lib, **kw) == code


def decode_one(lib, q=A, kc=A, vc=A, sl=A2, o=A, lse=A2, ws=A, wn=1 << 30, B=2, Hq=8, Hkv=2,
               max_len=64, d=128, scale=0.1, dtype=0):
    return lib.attn_decode(q, kc, vc, sl, o, lse, ws, wn, B, Hq, Hkv, max_len, d, scale, dtype,
                           None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1), (dict(sl=None), -1),
    (dict(B=0), -2), (dict(max_len=0), -2), (dict(Hq=6, Hkv=4), -2), (dict(max_len=2**23 + 1), -2),
    (dict(d=80), -3), (dict(dtype=5), -3), (dict(Hq=66, Hkv=2), -3),
    (dict(scale=0.0), -5), (dict(kc=MIS), -4), (dict(ws=MIS), -4),
])
def test_attn_decode_rejects(lib, kw, code):
    assert decode_one(lib, **kw) == code


def test_attn_decode_workspace_rejects_bad_shapes(lib):
    assert lib.attn_decode_workspace(0, 8, 2, 64, 128) == -2
    assert lib.attn_decode_workspace(2, 8, 2, 64, 96) == -3
    assert lib.attn_decode_workspace(2, 6, 4, 64, 128) == -2


def fused(lib, q=A, kc=A, vc=A, sl=A2, o=A, lse=A2, ws=ctypes.c_void_p(1 << 20), wn=1 << 30,
          B=2, Hq=8, Hkv=2, max_len=64, d=128, chunk=16, scale=0.1, dtype=0):
    return lib.attn_decode_fused(q, kc, vc, sl, o, lse, ws, wn, B, Hq, Hkv, max_len, d, chunk,
                                 scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1), (dict(ws=None), -1),
    (dict(B=0), -2), (dict(max_len=0), -2), (dict(chunk=0), -2), (dict(Hq=6, Hkv=4), -2),
    (dict(max_len=2**23 + 1), -2),
    (dict(d=80), -3), (dict(dtype=5), -3), (dict(Hq=66, Hkv=2), -3),
    # one pair's partials span (Hq/Hkv) * C * d * 4 bytes, which must stay below 2^32
    (dict(Hq=64, Hkv=2, max_len=2**23, chunk=16), -3),
    (dict(scale=0.0), -5), (dict(kc=MIS), -4), (dict(ws=ctypes.c_void_p(4096 + 128)), -4),
    (dict(wn=100), -5),
])
def test_attn_decode_fused_rejects(lib, kw, code):
    assert fused(lib, **kw) == code


def test_attn_decode_fused_workspace_layout(lib):
    # counters [B*Hkv] and part_lse [B*Hq*C] each padded to 64 words, then part_o
    up = lambda n: -(-n // 64) * 64
    for B, Hq, Hkv, L, d, chunk in [(64, 32, 8, 32768, 128, 512), (3, 4, 1, 100, 64, 7),
                                     (1, 1, 1, 1, 64, 1)]:
        C = -(-L // chunk)
        want = up(B * Hkv) + up(B * Hq * C) + B * Hq * C * d
        assert lib.attn_decode_fused_workspace(B, Hq, Hkv, L, d, chunk) == want
    assert lib.attn_decode_fused_workspace(0, 8, 2, 64, 128, 16) == -2
    assert lib.attn_decode_fused_workspace(2, 8, 2, 64, 96, 16) == -3
    assert lib.attn_decode_fused_workspace(2, 8, 2, 64, 128, 0) == -2


def fused_paged(lib, q=A, kp=A, vp=A, bt=A2, sl=A2, o=A, lse=A2, ws=ctypes.c_void_p(1 << 20),
                wn=1 << 30, B=2, Hq=8, Hkv=2, num_pages=10, page_size=32, max_pages=4, d=128,
                chunk=64, scale=0.1, dtype=0):
    return lib.attn_decode_fused_paged(q, kp, vp, bt, sl, o, lse, ws, wn, B, Hq, Hkv, num_pages,
                                       page_size, max_pages, d, chunk, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(bt=None), -1), (dict(ws=None), -1),
    (dict(B=0), -2), (dict(num_pages=0), -2), (dict(page_size=0), -2), (dict(max_pages=0), -2),
    (dict(chunk=0), -2), (dict(max_pages=2**18, page_size=64), -2),
    (dict(d=80), -3), (dict(page_size=24), -3), (dict(chunk=40), -3),
    (dict(page_size=16, chunk=512), -3),
    (dict(scale=float("nan")), -5), (dict(vp=MIS), -4), (dict(bt=ctypes.c_void_p(4098)), -4),
    (dict(wn=10), -5),
])
def test_attn_decode_fused_paged_rejects(lib, kw, code):
    assert fused_paged(lib, **kw) == code


def combine(lib, po=A, pl=A2, sl=A2, o=A, lse=A2, B=2, Hq=8, C=4, d=128, chunk=16, dtype=0):
    return lib.attn_decode_combine(po, pl, sl, o, lse, B, Hq, C, d, chunk, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(po=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(C=0), -2), (dict(chunk=-3), -2),
    (dict(d=32), -3), (dict(dtype=-1), -3), (dict(po=MIS), -4), (dict(o=MIS), -4),
])
def test_attn_decode_combine_rejects(lib, kw, code):
    assert combine(lib, **kw) == code


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        ea.fwd(q, q, q)
