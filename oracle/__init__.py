"""Exact fp64 CPU attention oracle (ctypes wrapper over ``attn_oracle.c``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. The GPU library does not
import it and shares no code with it.

Every function takes 16-bit float patterns as ``numpy.uint16`` arrays (bf16 when
``dtype == 0``, IEEE fp16 when ``dtype == 1``) and returns ``numpy.float64``
arrays. What each one computes is documented in ``attn_oracle.c``: the plain
definition of attention, materialising each row's score vector in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A build instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
# (any out-of-bounds access, use after free or undefined operation aborts).
# Loading it needs the ASan runtime first in the process (LD_PRELOAD), so the
# tests use it from a child process that sets ORACLE_LIB to its path.
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
_COMMON_FLAGS = ["-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                 "-fno-fast-math", "-ffp-contract=off"]

BF16 = 0
FP16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compiles ``attn_oracle.c`` with gcc (fp64, OpenMP) into ``liboracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2"] + _COMMON_FLAGS + [_SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized() -> str:
    """Compiles ``attn_oracle.c`` with -fsanitize=address,undefined (errors
    abort) into ``liboracle_san.so`` and returns its path."""
    tmp = _LIB_SAN + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"] + _COMMON_FLAGS + [_SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_SAN)
    return _LIB_SAN


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = build(force=False)
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i = ctypes.c_int
        i64 = ctypes.c_int64
        f = ctypes.c_float
        lib.oracle_attn_fwd.argtypes = [p, p, p, i, i, i, i, i, i, i, f, i, p, p, i]
        lib.oracle_attn_fwd_rows.argtypes = [p, p, p, i, i, i, i, i, i, i, f, i, p, i64, p, p, i]
        lib.oracle_attn_fwd_local.argtypes = [p, p, p, i, i, i, i, i, i, i, f, i, i, p, p, i]
        lib.oracle_attn_fwd_qkvpacked.argtypes = [p, i, i, i, i, i, f, i, p, p, i]
        lib.oracle_decode.argtypes = [p, p, p, p, i, i, i, i, i, i, f, p, p, i]
        lib.oracle_attn_bwd.argtypes = [p, p, p, p, i, i, i, i, i, i, i, f, i, p, p, p, i]
        lib.oracle_attn_fwd_varlen.argtypes = [p, p, p, p, p, i, i, i, i, i, i, i, f, i, p, p, i]
        lib.oracle_decode_paged.argtypes = [p, p, p, p, p, i, i, i, i, i, i, i, i, f, p, p, i]
        lib.oracle_decode_chunks.argtypes = [p, p, p, p, i, i, i, i, i, i, i, f, p, p, i]
        lib.oracle_combine.argtypes = [p, p, p, i, i, i, i, i, p, p]
        lib.oracle_decode_values.argtypes = [p, i64, i, p]
        lib.oracle_max_threads.argtypes = []
        for fn in (lib.oracle_attn_fwd, lib.oracle_attn_fwd_rows, lib.oracle_decode,
                   lib.oracle_decode_paged, lib.oracle_attn_fwd_varlen, lib.oracle_attn_bwd,
                   lib.oracle_attn_fwd_local, lib.oracle_attn_fwd_qkvpacked,
                   lib.oracle_decode_chunks, lib.oracle_combine, lib.oracle_decode_values,
                   lib.oracle_max_threads):
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected uint16 bit patterns, got %s" % a.dtype)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def max_threads() -> int:
    return _load().oracle_max_threads()


def decode_values(bits, dtype: int) -> np.ndarray:
    """Decodes 16-bit patterns to fp64 exactly."""
    bits = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _check(_load().oracle_decode_values(_ptr(bits), bits.size, dtype, _ptr(out)), "decode")
    return out


def attn_fwd(q, k, v, dtype: int, scale: float, causal: bool, nthreads: int = 0):
    """Exact attention: q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] -> (o [B,Hq,Nq,d], lse [B,Hq,Nq])."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch")
    o = np.empty((B, Hq, Nq, d), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    rc = _load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), dtype, B, Hq, Hkv, Nq, Nk, d,
                                 float(scale), int(bool(causal)), _ptr(o), _ptr(lse), nthreads)
    _check(rc, "attn_fwd")
    return o, lse


def attn_fwd_qkvpacked(qkv, dtype: int, scale: float, causal: bool, nthreads: int = 0):
    """Attention from a packed qkv [B,N,3,H,d] -> (o [B,N,H,d], lse [B,H,N])."""
    qkv = _u16(qkv)
    if qkv.ndim != 5 or qkv.shape[2] != 3:
        raise ValueError("qkv must be [B,N,3,H,d]")
    B, N, _, H, d = qkv.shape
    o = np.empty((B, N, H, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    rc = _load().oracle_attn_fwd_qkvpacked(_ptr(qkv), dtype, B, N, H, d, float(scale),
                                           int(bool(causal)), _ptr(o), _ptr(lse), nthreads)
    _check(rc, "attn_fwd_qkvpacked")
    return o, lse


def attn_fwd_local(q, k, v, dtype: int, scale: float, window_left: int, window_right: int,
                   nthreads: int = 0):
    """Sliding-window attention (negative bound = none) -> (o [B,Hq,Nq,d], lse [B,Hq,Nq])."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch")
    o = np.empty((B, Hq, Nq, d), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    rc = _load().oracle_attn_fwd_local(_ptr(q), _ptr(k), _ptr(v), dtype, B, Hq, Hkv, Nq, Nk, d,
                                       float(scale), int(window_left), int(window_right), _ptr(o),
                                       _ptr(lse), nthreads)
    _check(rc, "attn_fwd_local")
    return o, lse


def attn_fwd_rows(q, k, v, dtype: int, scale: float, causal: bool, rows, nthreads: int = 0):
    """Exact attention for selected rows; rows is an int64 array [n, 3] of (b, h, i)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v), dtype, B, Hq, Hkv, Nq, Nk, d,
                                      float(scale), int(bool(causal)), _ptr(rows), n, _ptr(o),
                                      _ptr(lse), nthreads)
    _check(rc, "attn_fwd_rows")
    return o, lse


def attn_bwd(q, k, v, dout, dtype: int, scale: float, causal: bool, nthreads: int = 0):
    """Gradients of sum(dout * O) for O = attention(q, k, v): q/dout [B,Hq,Nq,d], k/v
    [B,Hkv,Nk,d] -> (dq, dk, dv) fp64 of the same shapes."""
    q, k, v, do = _u16(q), _u16(k), _u16(v), _u16(dout)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk_ = k.shape
    if v.shape != k.shape or do.shape != q.shape or Bk != B or dk_ != d:
        raise ValueError("shape mismatch")
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(k.shape, dtype=np.float64)
    rc = _load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), dtype, B, Hq, Hkv, Nq, Nk,
                                 d, float(scale), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv),
                                 nthreads)
    _check(rc, "attn_bwd")
    return dq, dk, dv


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, dtype: int, scale: float, causal: bool,
                    nthreads: int = 0):
    """Exact attention over a packed batch: q [total_q,Hq,d], k/v [total_k,Hkv,d], cu_seqlens
    [B+1] -> (o [total_q,Hq,d], lse [Hq,total_q])."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    cq = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    ck = np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    if v.shape != k.shape or dk != d or cq.shape != ck.shape or cq.ndim != 1:
        raise ValueError("shape mismatch")
    o = np.empty((total_q, Hq, d), dtype=np.float64)
    lse = np.empty((Hq, total_q), dtype=np.float64)
    rc = _load().oracle_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cq), _ptr(ck), dtype,
                                        cq.shape[0] - 1, Hq, Hkv, total_q, total_k, d,
                                        float(scale), int(bool(causal)), _ptr(o), _ptr(lse),
                                        nthreads)
    _check(rc, "attn_fwd_varlen")
    return o, lse


def decode(q, k_cache, v_cache, seq_lens, dtype: int, scale: float, nthreads: int = 0):
    """Single-token decode: q [B,Hq,d], caches [B,Hkv,max_len,d] -> (o [B,Hq,d], lse [B,Hq])."""
    q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, d = q.shape
    _, Hkv, max_len, _ = kc.shape
    o = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = _load().oracle_decode(_ptr(q), _ptr(kc), _ptr(vc), _ptr(sl), dtype, B, Hq, Hkv,
                               max_len, d, float(scale), _ptr(o), _ptr(lse), nthreads)
    _check(rc, "decode")
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, dtype: int, scale: float,
                 nthreads: int = 0):
    """Single-token decode over a paged cache: q [B,Hq,d], pages [num_pages,page_size,Hkv,d],
    block_table [B,max_pages] int32 -> (o [B,Hq,d], lse [B,Hq])."""
    q, kp, vp = _u16(q), _u16(k_pages), _u16(v_pages)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = kp.shape
    if vp.shape != kp.shape or dk != d or bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("shape mismatch")
    o = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = _load().oracle_decode_paged(_ptr(q), _ptr(kp), _ptr(vp), _ptr(bt), _ptr(sl), dtype, B,
                                     Hq, Hkv, num_pages, page_size, bt.shape[1], d,
                                     float(scale), _ptr(o), _ptr(lse), nthreads)
    _check(rc, "decode_paged")
    return o, lse


def decode_chunks(q, k_cache, v_cache, seq_lens, dtype: int, chunk: int, scale: float,
                  nthreads: int = 0):
    """Per-chunk exact partials -> (part_o [B,Hq,C,d], part_lse [B,Hq,C])."""
    q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, d = q.shape
    _, Hkv, max_len, _ = kc.shape
    C = (max_len + chunk - 1) // chunk
    po = np.empty((B, Hq, C, d), dtype=np.float64)
    pl = np.empty((B, Hq, C), dtype=np.float64)
    rc = _load().oracle_decode_chunks(_ptr(q), _ptr(kc), _ptr(vc), _ptr(sl), dtype, B, Hq, Hkv,
                                      max_len, d, chunk, float(scale), _ptr(po), _ptr(pl),
                                      nthreads)
    _check(rc, "decode_chunks")
    return po, pl


def combine(part_o, part_lse, seq_lens, chunk: int):
    """Merges chunk partials (any float dtype, widened to fp64) -> (o [B,Hq,d], lse [B,Hq])."""
    po = np.ascontiguousarray(part_o, dtype=np.float64)
    pl = np.ascontiguousarray(part_lse, dtype=np.float64)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, C, d = po.shape
    o = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = _load().oracle_combine(_ptr(po), _ptr(pl), _ptr(sl), B, Hq, C, d, chunk, _ptr(o),
                                _ptr(lse))
    _check(rc, "combine")
    return o, lse
