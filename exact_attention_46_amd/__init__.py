"""MI355X-native exact attention: fused forward with LSE (dense or packed
variable-length batches) and split-KV decode (contiguous or paged KV cache).

The compute runs in hand-written HIP kernels for gfx950 behind a C ABI
(``include/mi355attn.h``, built into ``libmi355attn.so``); this package is the
thin Python binding over it. The library is loaded on first use and there is
no CPU fallback.
"""
from ._binding import (  # noqa: F401
    AttnError,
    bwd,
    EXPORTS,
    LIB_PATH,
    attn_bwd,
    attn_bwd_noalloc,
    attn_bwd_ds,
    attn_bwd_ds_workspace,
    bwd_ds,
    ds_workspace,
    attn_decode,
    attn_decode_combine,
    attn_decode_fused,
    attn_decode_fused_paged,
    attn_decode_fused_workspace,
    attn_decode_split,
    attn_decode_split_paged,
    attn_decode_workspace,
    attn_fwd,
    attn_fwd_local,
    attn_fwd_qkvpacked,
    attn_fwd_varlen,
    attn_status_str,
    decode,
    decode_auto,
    decode_buffers,
    decode_fused,
    decode_paged,
    default_scale,
    fwd,
    fwd_local,
    fwd_qkvpacked,
    fwd_varlen,
    fused_workspace,
    load_library,
)
