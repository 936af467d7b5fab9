"""ctypes binding of ``libmi355attn.so``: argument marshalling only.

The functions with the C names (``attn_fwd``, ``attn_decode_split``,
``attn_decode_combine``, ``attn_status_str``) take torch tensors that already
live on the GPU, check that they match the C contract (device, dtype,
contiguity, shapes), pass their device pointers and torch's current HIP stream,
and raise ``AttnError`` on a non-zero status. ``fwd`` and ``decode`` also
allocate the outputs. Every step of the computation runs in the HIP kernels;
nothing here computes attention, and there is no CPU fallback: if the library
is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmi355attn.so")

OK = 0
ERR_NULL_PTR = -1
ERR_BAD_SHAPE = -2
ERR_UNSUPPORTED = -3
ERR_MISALIGNED = -4
ERR_BAD_ARG = -5
ERR_HIP = -6
ERR_SCRATCH = -7

EXPORTS = ("attn_fwd", "attn_fwd_varlen", "attn_fwd_local", "attn_fwd_qkvpacked", "attn_bwd",
           "attn_bwd_noalloc", "attn_bwd_ds", "attn_bwd_ds_workspace",
           "attn_decode_split",
           "attn_decode_split_paged", "attn_decode_combine", "attn_decode",
           "attn_decode_workspace", "attn_decode_fused", "attn_decode_fused_paged",
           "attn_decode_fused_workspace", "attn_status_str")

_DTYPE_CODE = {torch.bfloat16: 0, torch.float16: 1}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed with status %d: %s" % (fn, status, attn_status_str(status)))
        self.status = status


def load_library() -> ctypes.CDLL:
    """Loads the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmi355attn.so is not built (run python -m "
                               "exact_attention_46_amd.build); there is no fallback")
        lib = ctypes.CDLL(LIB_PATH)
        p, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        ll = ctypes.c_longlong
        lib.attn_fwd.argtypes = [p, p, p, p, p, i, i, i, i, i, i, f, i, i, p]
        lib.attn_fwd_varlen.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, i, i, f, i, i, p]
        lib.attn_fwd_local.argtypes = [p, p, p, p, p, i, i, i, i, i, i, f, i, i, i, p]
        lib.attn_fwd_qkvpacked.argtypes = [p, p, p, i, i, i, i, f, i, i, p]
        lib.attn_bwd.argtypes = [p, p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, f, i, i, p]
        lib.attn_bwd_noalloc.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, f, i, i, p]
        lib.attn_bwd_ds.argtypes = [p, p, p, p, p, p, p, p, ll, p, p, p, i, i, i, i, i, i, f, i, i,
                                    p]
        lib.attn_bwd_ds_workspace.argtypes = [i, i, i, i]
        lib.attn_decode.argtypes = [p, p, p, p, p, p, p, ll, i, i, i, i, i, f, i, p]
        lib.attn_decode_workspace.argtypes = [i, i, i, i, i]
        lib.attn_decode_split.argtypes = [p, p, p, p, p, p, i, i, i, i, i, i, f, i, p]
        lib.attn_decode_split_paged.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, i, i, i, f,
                                                i, p]
        lib.attn_decode_combine.argtypes = [p, p, p, p, p, i, i, i, i, i, i, p]
        lib.attn_decode_fused.argtypes = [p, p, p, p, p, p, p, ll, i, i, i, i, i, i, f, i, p]
        lib.attn_decode_fused_paged.argtypes = [p, p, p, p, p, p, p, p, ll, i, i, i, i, i, i, i,
                                                i, f, i, p]
        lib.attn_decode_fused_workspace.argtypes = [i, i, i, i, i, i]
        lib.attn_status_str.argtypes = [i]
        lib.attn_fwd.restype = i
        lib.attn_fwd_varlen.restype = i
        lib.attn_fwd_local.restype = i
        lib.attn_fwd_qkvpacked.restype = i
        lib.attn_bwd.restype = i
        lib.attn_bwd_noalloc.restype = i
        lib.attn_bwd_ds.restype = i
        lib.attn_bwd_ds_workspace.restype = ctypes.c_longlong
        lib.attn_decode.restype = i
        lib.attn_decode_workspace.restype = ctypes.c_longlong
        lib.attn_decode_split.restype = i
        lib.attn_decode_split_paged.restype = i
        lib.attn_decode_combine.restype = i
        lib.attn_decode_fused.restype = i
        lib.attn_decode_fused_paged.restype = i
        lib.attn_decode_fused_workspace.restype = ctypes.c_longlong
        lib.attn_status_str.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _gpu(*ts):
    for t in ts:
        _need(t.is_cuda, "tensors must be on the GPU (no CPU path exists)")
        _need(t.is_contiguous(), "tensors must be contiguous")


def _dtype_code(t: torch.Tensor) -> int:
    _need(t.dtype in _DTYPE_CODE, "q/k/v must be bfloat16 or float16")
    return _DTYPE_CODE[t.dtype]


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def attn_fwd(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """Calls attn_fwd. q/o [B,Hq,Nq,d], k/v [B,Hkv,Nk,d], lse [B,Hq,Nq] fp32."""
    _gpu(q, k, v, o, lse)
    _need(q.dim() == 4 and k.dim() == 4 and v.shape == k.shape, "q, k, v must be 4-D, k ~ v")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _need(k.shape[0] == B and k.shape[3] == d, "k/v batch or head dim differ from q")
    _need(k.dtype == q.dtype and v.dtype == q.dtype and o.dtype == q.dtype, "dtypes differ")
    _need(o.shape == q.shape, "o must have q's shape")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, Hq, Nq), "lse [B,Hq,Nq] fp32")
    st = load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq,
                                 Nk, d, float(scale), int(bool(causal)), _dtype_code(q),
                                 _stream(stream))
    if st != OK:
        raise AttnError("attn_fwd", st)


def attn_fwd_qkvpacked(qkv, o, lse, causal: bool, scale: float, stream=None) -> None:
    """Calls attn_fwd_qkvpacked. qkv [B,N,3,H,d]; o [B,N,H,d]; lse [B,H,N] fp32."""
    _gpu(qkv, o, lse)
    _need(qkv.dim() == 5 and qkv.shape[2] == 3, "qkv must be [B,N,3,H,d]")
    B, N, _, H, d = qkv.shape
    _need(o.dtype == qkv.dtype and tuple(o.shape) == (B, N, H, d), "o [B,N,H,d]")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, N), "lse [B,H,N] fp32")
    st = load_library().attn_fwd_qkvpacked(_ptr(qkv), _ptr(o), _ptr(lse), B, N, H, d,
                                           float(scale), int(bool(causal)), _dtype_code(qkv),
                                           _stream(stream))
    if st != OK:
        raise AttnError("attn_fwd_qkvpacked", st)


def fwd_qkvpacked(qkv, causal: bool = True, scale: float | None = None, stream=None):
    """Allocates and returns (o [B,N,H,d], lse [B,H,N]) for a packed qkv tensor."""
    B, N, _, H, d = qkv.shape
    if scale is None:
        scale = default_scale(d)
    o = torch.empty((B, N, H, d), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=qkv.device)
    attn_fwd_qkvpacked(qkv, o, lse, causal, scale, stream)
    return o, lse


def attn_fwd_local(q, k, v, o, lse, window_left: int, window_right: int, scale: float,
                   stream=None) -> None:
    """Calls attn_fwd_local (shapes as attn_fwd; a negative window bound is no bound)."""
    _gpu(q, k, v, o, lse)
    _need(q.dim() == 4 and k.dim() == 4 and v.shape == k.shape, "q, k, v must be 4-D, k ~ v")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _need(k.shape[0] == B and k.shape[3] == d, "k/v batch or head dim differ from q")
    _need(k.dtype == q.dtype and v.dtype == q.dtype and o.dtype == q.dtype, "dtypes differ")
    _need(o.shape == q.shape, "o must have q's shape")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, Hq, Nq), "lse [B,Hq,Nq] fp32")
    st = load_library().attn_fwd_local(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                       Nq, Nk, d, float(scale), int(window_left),
                                       int(window_right), _dtype_code(q), _stream(stream))
    if st != OK:
        raise AttnError("attn_fwd_local", st)


def fwd_local(q, k, v, window_left: int, window_right: int = 0, scale: float | None = None,
              stream=None):
    """Allocates and returns (o, lse) for sliding-window attention."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_local(q, k, v, o, lse, window_left, window_right, scale, stream)
    return o, lse


def attn_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, causal: bool, scale: float,
             stream=None) -> None:
    """Calls attn_bwd. q/o/dout/dq [B,Hq,Nq,d]; k/v/dk/dv [B,Hkv,Nk,d]; lse and the
    workspace delta [B,Hq,Nq] fp32."""
    _gpu(q, k, v, o, dout, lse, delta, dq, dk, dv)
    _need(q.dim() == 4 and k.dim() == 4 and v.shape == k.shape, "q, k, v must be 4-D, k ~ v")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _need(k.shape[0] == B and k.shape[3] == d, "k/v batch or head dim differ from q")
    for t in (k, v, o, dout, dq, dk, dv):
        _need(t.dtype == q.dtype, "dtypes differ")
    _need(o.shape == q.shape and dout.shape == q.shape and dq.shape == q.shape,
          "o, dout, dq must have q's shape")
    _need(dk.shape == k.shape and dv.shape == k.shape, "dk, dv must have k's shape")
    for t in (lse, delta):
        _need(t.dtype == torch.float32 and tuple(t.shape) == (B, Hq, Nq), "lse/delta [B,Hq,Nq] fp32")
    st = load_library().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                 _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nk, d,
                                 float(scale), int(bool(causal)), _dtype_code(q), _stream(stream))
    if st != OK:
        raise AttnError("attn_bwd", st)


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal: bool, scale: float,
                     stream=None) -> None:
    """Calls attn_bwd_noalloc: attn_bwd with D in the library's fixed scratch (no
    delta argument, nothing allocated; B*Hq*Nq at most 4194304)."""
    _gpu(q, k, v, o, dout, lse, dq, dk, dv)
    _need(q.dim() == 4 and k.dim() == 4 and v.shape == k.shape, "q, k, v must be 4-D, k ~ v")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _need(k.shape[0] == B and k.shape[3] == d, "k/v batch or head dim differ from q")
    for t in (k, v, o, dout, dq, dk, dv):
        _need(t.dtype == q.dtype, "dtypes differ")
    _need(o.shape == q.shape and dout.shape == q.shape and dq.shape == q.shape,
          "o, dout, dq must have q's shape")
    _need(dk.shape == k.shape and dv.shape == k.shape, "dk, dv must have k's shape")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, Hq, Nq), "lse [B,Hq,Nq] fp32")
    st = load_library().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                         _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq,
                                         Nk, d, float(scale), int(bool(causal)), _dtype_code(q),
                                         _stream(stream))
    if st != OK:
        raise AttnError("attn_bwd_noalloc", st)


def attn_bwd_ds_workspace(B: int, Hq: int, Nq: int, Nk: int) -> int:
    """Bytes of the dS^T workspace attn_bwd_ds needs (raises on a bad shape)."""
    n = load_library().attn_bwd_ds_workspace(B, Hq, Nq, Nk)
    if n < 0:
        raise AttnError("attn_bwd_ds_workspace", int(n))
    return int(n)


def ds_workspace(q, k) -> torch.Tensor:
    """A dS^T workspace for attn_bwd_ds (uninitialised bytes; 256-byte aligned)."""
    B, Hq, Nq, _ = q.shape
    n = attn_bwd_ds_workspace(B, Hq, Nq, k.shape[2])
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def attn_bwd_ds(q, k, v, o, dout, lse, delta, ds, dq, dk, dv, causal: bool, scale: float,
                stream=None) -> None:
    """Calls attn_bwd_ds: attn_bwd with dS stored once in the workspace `ds` (a uint8
    tensor of at least attn_bwd_ds_workspace bytes) instead of recomputed."""
    _gpu(q, k, v, o, dout, lse, delta, ds, dq, dk, dv)
    _need(q.dim() == 4 and k.dim() == 4 and v.shape == k.shape, "q, k, v must be 4-D, k ~ v")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _need(k.shape[0] == B and k.shape[3] == d, "k/v batch or head dim differ from q")
    for t in (k, v, o, dout, dq, dk, dv):
        _need(t.dtype == q.dtype, "dtypes differ")
    _need(o.shape == q.shape and dout.shape == q.shape and dq.shape == q.shape,
          "o, dout, dq must have q's shape")
    _need(dk.shape == k.shape and dv.shape == k.shape, "dk, dv must have k's shape")
    for t in (lse, delta):
        _need(t.dtype == torch.float32 and tuple(t.shape) == (B, Hq, Nq), "lse/delta [B,Hq,Nq] fp32")
    _need(ds.is_contiguous(), "ds must be contiguous")
    st = load_library().attn_bwd_ds(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                    _ptr(delta), _ptr(ds), ds.numel() * ds.element_size(),
                                    _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nk, d,
                                    float(scale), int(bool(causal)), _dtype_code(q),
                                    _stream(stream))
    if st != OK:
        raise AttnError("attn_bwd_ds", st)


def bwd_ds(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None,
           stream=None, ds=None):
    """Allocates (unless `ds` is given) and returns (dq, dk, dv) through attn_bwd_ds."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if ds is None:
        ds = ds_workspace(q, k)
    attn_bwd_ds(q, k, v, o, dout, lse, delta, ds, dq, dk, dv, causal, scale, stream)
    return dq, dk, dv


def bwd(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None, stream=None):
    """Allocates and returns (dq, dk, dv) for attention backward."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, causal, scale, stream)
    return dq, dk, dv


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                    causal: bool, scale: float, stream=None) -> None:
    """Calls attn_fwd_varlen. q/o [total_q,Hq,d], k/v [total_k,Hkv,d], lse [Hq,total_q] fp32,
    cu_seqlens_q/k [B+1] int32 on the GPU."""
    _gpu(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k)
    _need(q.dim() == 3 and k.dim() == 3 and v.shape == k.shape, "q, k, v must be 3-D, k ~ v")
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    _need(k.shape[2] == d, "k/v head dim differs from q")
    _need(k.dtype == q.dtype and v.dtype == q.dtype and o.dtype == q.dtype, "dtypes differ")
    _need(o.shape == q.shape, "o must have q's shape")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (Hq, total_q), "lse [Hq,total_q] fp32")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32 and
          cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape == cu_seqlens_k.shape and
          cu_seqlens_q.shape[0] >= 2, "cu_seqlens_q/k [B+1] int32")
    B = cu_seqlens_q.shape[0] - 1
    st = load_library().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Hq, Hkv,
                                        total_q, total_k, int(max_seqlen_q), d, float(scale),
                                        int(bool(causal)), _dtype_code(q), _stream(stream))
    if st != OK:
        raise AttnError("attn_fwd_varlen", st)


def attn_decode_split(q, k_cache, v_cache, seq_lens, part_o, part_lse, chunk: int,
                      scale: float, stream=None) -> None:
    """Calls attn_decode_split. q [B,Hq,d], caches [B,Hkv,max_len,d], seq_lens [B] int32,
    part_o [B,Hq,C,d] fp32, part_lse [B,Hq,C] fp32 with C = ceil(max_len/chunk)."""
    _gpu(q, k_cache, v_cache, seq_lens, part_o, part_lse)
    B, Hq, d = q.shape
    _, Hkv, max_len, _ = k_cache.shape
    _need(v_cache.shape == k_cache.shape and k_cache.shape[0] == B and k_cache.shape[3] == d,
          "cache shapes")
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "dtypes differ")
    _need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,), "seq_lens [B] int32")
    C = -(-max_len // chunk)
    _need(part_o.dtype == torch.float32 and tuple(part_o.shape) == (B, Hq, C, d), "part_o shape")
    _need(part_lse.dtype == torch.float32 and tuple(part_lse.shape) == (B, Hq, C),
          "part_lse shape")
    st = load_library().attn_decode_split(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                          _ptr(part_o), _ptr(part_lse), B, Hq, Hkv, max_len, d,
                                          int(chunk), float(scale), _dtype_code(q),
                                          _stream(stream))
    if st != OK:
        raise AttnError("attn_decode_split", st)


def attn_decode_split_paged(q, k_pages, v_pages, block_table, seq_lens, part_o, part_lse,
                            chunk: int, scale: float, stream=None) -> None:
    """Calls attn_decode_split_paged. q [B,Hq,d]; pages [num_pages,page_size,Hkv,d];
    block_table [B,max_pages] int32; part_o [B,Hq,C,d], part_lse [B,Hq,C] fp32 with
    C = ceil(max_pages*page_size/chunk)."""
    _gpu(q, k_pages, v_pages, block_table, seq_lens, part_o, part_lse)
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, _ = k_pages.shape
    _need(v_pages.shape == k_pages.shape and k_pages.shape[3] == d, "page shapes")
    _need(k_pages.dtype == q.dtype and v_pages.dtype == q.dtype, "dtypes differ")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and
          block_table.shape[0] == B, "block_table [B,max_pages] int32")
    _need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,), "seq_lens [B] int32")
    max_pages = block_table.shape[1]
    C = -(-(max_pages * page_size) // chunk)
    _need(part_o.dtype == torch.float32 and tuple(part_o.shape) == (B, Hq, C, d), "part_o shape")
    _need(part_lse.dtype == torch.float32 and tuple(part_lse.shape) == (B, Hq, C),
          "part_lse shape")
    st = load_library().attn_decode_split_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), _ptr(part_o),
        _ptr(part_lse), B, Hq, Hkv, num_pages, page_size, max_pages, d, int(chunk), float(scale),
        _dtype_code(q), _stream(stream))
    if st != OK:
        raise AttnError("attn_decode_split_paged", st)


def attn_decode_combine(part_o, part_lse, seq_lens, o, lse, chunk: int, stream=None) -> None:
    """Calls attn_decode_combine. o [B,Hq,d] bf16/fp16, lse [B,Hq] fp32."""
    _gpu(part_o, part_lse, seq_lens, o, lse)
    B, Hq, C, d = part_o.shape
    _need(o.dtype in _DTYPE_CODE and tuple(o.shape) == (B, Hq, d), "o [B,Hq,d] bf16/fp16")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, Hq), "lse [B,Hq] fp32")
    _need(tuple(part_lse.shape) == (B, Hq, C), "part_lse shape")
    st = load_library().attn_decode_combine(_ptr(part_o), _ptr(part_lse), _ptr(seq_lens),
                                            _ptr(o), _ptr(lse), B, Hq, C, d, int(chunk),
                                            _DTYPE_CODE[o.dtype], _stream(stream))
    if st != OK:
        raise AttnError("attn_decode_combine", st)


def fwd(q, k, v, causal: bool = True, scale: float | None = None, stream=None):
    """Allocates and returns (o, lse) for attention forward."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = True,
               scale: float | None = None, stream=None):
    """Allocates and returns (o [total_q,Hq,d], lse [Hq,total_q]) for a packed batch."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal, scale,
                    stream)
    return o, lse


def decode_buffers(q, max_len: int, chunk: int):
    """Allocates (part_o, part_lse, o, lse) for a decode of q [B,Hq,d]."""
    B, Hq, d = q.shape
    C = -(-max_len // chunk)
    part_o = torch.empty((B, Hq, C, d), dtype=torch.float32, device=q.device)
    part_lse = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    o = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    return part_o, part_lse, o, lse


def decode(q, k_cache, v_cache, seq_lens, chunk: int = 512, scale: float | None = None,
           stream=None, buffers=None):
    """Split-KV decode: split then combine on the same stream. Returns (o, lse)."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    if buffers is None:
        buffers = decode_buffers(q, k_cache.shape[2], chunk)
    part_o, part_lse, o, lse = buffers
    attn_decode_split(q, k_cache, v_cache, seq_lens, part_o, part_lse, chunk, scale, stream)
    attn_decode_combine(part_o, part_lse, seq_lens, o, lse, chunk, stream)
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, chunk: int = 512,
                 scale: float | None = None, stream=None, buffers=None):
    """Split-KV decode over a paged cache: split then combine. Returns (o, lse)."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    if buffers is None:
        buffers = decode_buffers(q, block_table.shape[1] * k_pages.shape[1], chunk)
    part_o, part_lse, o, lse = buffers
    attn_decode_split_paged(q, k_pages, v_pages, block_table, seq_lens, part_o, part_lse, chunk,
                            scale, stream)
    attn_decode_combine(part_o, part_lse, seq_lens, o, lse, chunk, stream)
    return o, lse


def attn_decode_workspace(B: int, Hq: int, Hkv: int, max_len: int, d: int) -> int:
    """Floats of workspace attn_decode needs (0 for a single pass); raises on a bad shape."""
    n = load_library().attn_decode_workspace(B, Hq, Hkv, max_len, d)
    if n < 0:
        raise AttnError("attn_decode_workspace", int(n))
    return int(n)


def attn_decode(q, k_cache, v_cache, seq_lens, o, lse, workspace, scale: float,
                stream=None) -> None:
    """Calls attn_decode. workspace: fp32 tensor on the GPU (or None when none is needed)."""
    ts = [q, k_cache, v_cache, seq_lens, o, lse] + ([workspace] if workspace is not None else [])
    _gpu(*ts)
    B, Hq, d = q.shape
    _, Hkv, max_len, _ = k_cache.shape
    _need(v_cache.shape == k_cache.shape and k_cache.shape[0] == B and k_cache.shape[3] == d,
          "cache shapes")
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype and o.dtype == q.dtype,
          "dtypes differ")
    _need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,), "seq_lens [B] int32")
    _need(tuple(o.shape) == (B, Hq, d), "o [B,Hq,d]")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, Hq), "lse [B,Hq] fp32")
    if workspace is not None:
        _need(workspace.dtype == torch.float32, "workspace must be fp32")
    wp = _ptr(workspace) if workspace is not None else None
    wn = workspace.numel() if workspace is not None else 0
    st = load_library().attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                    _ptr(o), _ptr(lse), wp, wn, B, Hq, Hkv, max_len, d,
                                    float(scale), _dtype_code(q), _stream(stream))
    if st != OK:
        raise AttnError("attn_decode", st)


def decode_auto(q, k_cache, v_cache, seq_lens, scale: float | None = None, stream=None,
                workspace=None):
    """One-call decode with the library's chunk choice. Returns (o, lse)."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    B, Hq, d = q.shape
    if workspace is None:
        n = attn_decode_workspace(B, Hq, k_cache.shape[1], k_cache.shape[2], d)
        workspace = torch.empty((n,), dtype=torch.float32, device=q.device) if n else None
    o = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    attn_decode(q, k_cache, v_cache, seq_lens, o, lse, workspace, scale, stream)
    return o, lse


def attn_decode_fused_workspace(B: int, Hq: int, Hkv: int, max_len: int, d: int,
                                chunk: int) -> int:
    """Floats of workspace attn_decode_fused needs; raises on a rejected shape."""
    n = load_library().attn_decode_fused_workspace(B, Hq, Hkv, max_len, d, chunk)
    if n < 0:
        raise AttnError("attn_decode_fused_workspace", int(n))
    return int(n)


def fused_workspace(B: int, Hq: int, Hkv: int, max_len: int, d: int, chunk: int, device="cuda"):
    """A zeroed workspace for attn_decode_fused (its counters must start at zero;
    the kernel leaves them zero, so the tensor can be reused call after call)."""
    n = attn_decode_fused_workspace(B, Hq, Hkv, max_len, d, chunk)
    return torch.zeros((n,), dtype=torch.float32, device=device)


def _check_workspace(workspace):
    _need(workspace.dtype == torch.float32 and workspace.dim() == 1, "workspace: 1-D fp32")
    _need(workspace.data_ptr() % 256 == 0, "workspace must be 256-byte aligned")


def attn_decode_fused(q, k_cache, v_cache, seq_lens, o, lse, workspace, chunk: int,
                      scale: float, stream=None) -> None:
    """Calls attn_decode_fused. q [B,Hq,d], caches [B,Hkv,max_len,d], seq_lens [B] int32,
    o [B,Hq,d], lse [B,Hq] fp32, workspace from fused_workspace()."""
    _gpu(q, k_cache, v_cache, seq_lens, o, lse, workspace)
    B, Hq, d = q.shape
    _, Hkv, max_len, _ = k_cache.shape
    _need(v_cache.shape == k_cache.shape and k_cache.shape[0] == B and k_cache.shape[3] == d,
          "cache shapes")
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype and o.dtype == q.dtype,
          "dtypes differ")
    _need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,), "seq_lens [B] int32")
    _need(tuple(o.shape) == (B, Hq, d), "o [B,Hq,d]")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, Hq), "lse [B,Hq] fp32")
    _check_workspace(workspace)
    st = load_library().attn_decode_fused(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                          _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
                                          B, Hq, Hkv, max_len, d, int(chunk), float(scale),
                                          _dtype_code(q), _stream(stream))
    if st != OK:
        raise AttnError("attn_decode_fused", st)


def attn_decode_fused_paged(q, k_pages, v_pages, block_table, seq_lens, o, lse, workspace,
                            chunk: int, scale: float, stream=None) -> None:
    """Calls attn_decode_fused_paged (pages and block_table as attn_decode_split_paged)."""
    _gpu(q, k_pages, v_pages, block_table, seq_lens, o, lse, workspace)
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, _ = k_pages.shape
    _need(v_pages.shape == k_pages.shape and k_pages.shape[3] == d, "page shapes")
    _need(k_pages.dtype == q.dtype and v_pages.dtype == q.dtype and o.dtype == q.dtype,
          "dtypes differ")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and
          block_table.shape[0] == B, "block_table [B,max_pages] int32")
    _need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,), "seq_lens [B] int32")
    _need(tuple(o.shape) == (B, Hq, d), "o [B,Hq,d]")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (B, Hq), "lse [B,Hq] fp32")
    _check_workspace(workspace)
    st = load_library().attn_decode_fused_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), _ptr(o),
        _ptr(lse), _ptr(workspace), workspace.numel(), B, Hq, Hkv, num_pages, page_size,
        block_table.shape[1], d, int(chunk), float(scale), _dtype_code(q), _stream(stream))
    if st != OK:
        raise AttnError("attn_decode_fused_paged", st)


def decode_fused(q, k_cache, v_cache, seq_lens, chunk: int = 512, scale: float | None = None,
                 stream=None, workspace=None):
    """Split-KV decode with the combine fused into one launch. Returns (o, lse)."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    B, Hq, d = q.shape
    if workspace is None:
        workspace = fused_workspace(B, Hq, k_cache.shape[1], k_cache.shape[2], d, chunk, q.device)
    o = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    attn_decode_fused(q, k_cache, v_cache, seq_lens, o, lse, workspace, chunk, scale, stream)
    return o, lse
