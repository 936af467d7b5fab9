"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it contains none of the
attention arithmetic. Both the GPU path and the CPU oracle consume what it
returns (the oracle takes the raw 16-bit patterns of the same tensors).

Recipe (all draws from ``torch.Generator`` seeded with the workload's seed):
  * prefill: q, k, v drawn in that order as fp32 ``randn`` and cast to bf16/fp16
    with round-to-nearest-even;
  * long-context stress: after the three draws, for every (batch, kv-head) a
    ``randperm(Nk)`` picks round(0.01 * Nk) key rows whose fp32 values are scaled
    by 10 before the cast, which produces large-magnitude score outliers;
  * decode: the per-sequence lengths first (``randint`` on [l_min, l_max]), then
    q; the cache rows of sequence b at positions < L_b are drawn per sequence,
    k then v, and every cache row at a position >= L_b is filled with NaN so that
    any read past the end of a sequence shows up in the output. The cache draws
    use a generator on the device the cache lives on (a 4 GiB cache is too slow to
    draw on the host), so the values differ between a CPU and a GPU cache; the
    lengths and q never do;
  * paged decode: the rows of a padded decode cache are laid out in pages of
    ``page_size`` rows ([num_pages, page_size, Hkv, d]) at the positions of a
    seeded ``randperm`` of the pool, plus ``spare`` unused pages; every row no
    sequence uses (unused pages, the tail of each sequence's last page) is NaN,
    and unused block-table slots hold -1;
  * packed variable-length prefill: per-sequence query and key lengths given, q
    [total_q, Hq, d], k, v [total_k, Hkv, d] drawn in that order as fp32 ``randn``
    and cast; cu_seqlens are the running sums of the lengths.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
DTYPE_CODE = {"bf16": 0, "fp16": 1}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str
    seed: int
    causal: tuple = (True,)
    N: int = 0  # prefill: Nq == Nk == N
    l_min: int = 0  # decode only
    l_max: int = 0
    chunk: int = 512
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    notes: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


WORKLOADS = {
    "tiny": Workload("tiny", "prefill", B=1, Hq=2, Hkv=2, d=64, dtype="fp16", seed=0, N=128,
                     causal=(False, True)),
    "llm_prefill": Workload("llm_prefill", "prefill", B=4, Hq=32, Hkv=32, d=128, dtype="bf16",
                            seed=1, N=2048),
    "gqa_prefill": Workload("gqa_prefill", "prefill", B=2, Hq=32, Hkv=8, d=128, dtype="bf16",
                            seed=2, N=8192),
    "decode": Workload("decode", "decode", B=64, Hq=32, Hkv=8, d=128, dtype="bf16", seed=3,
                       l_min=512, l_max=32768, chunk=512),
    "long_context": Workload("long_context", "prefill", B=1, Hq=16, Hkv=16, d=128,
                             dtype="bf16", seed=4, N=32768, outlier_frac=0.01,
                             outlier_scale=10.0),
}


def prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", seed=0, outlier_frac=0.0,
                   outlier_scale=1.0):
    """Returns CPU tensors q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d] in ``dtype``."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((B, Hq, Nq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32)
    n_out = int(round(outlier_frac * Nk))
    if n_out > 0:
        for b in range(B):
            for h in range(Hkv):
                rows = torch.randperm(Nk, generator=g)[:n_out]
                k[b, h, rows] *= outlier_scale
    t = DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def outlier_rows(B, Hq, Hkv, Nq, Nk, d, seed, outlier_frac):
    """Replays the generator of ``prefill_inputs`` and returns the outlier key rows
    per (b, kv-head) as a list of lists of ints (used to pick rows to spot-check)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    torch.randn((B, Hq, Nq, d), generator=g, dtype=torch.float32)
    torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32)
    torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32)
    n_out = int(round(outlier_frac * Nk))
    out = []
    for b in range(B):
        per = []
        for h in range(Hkv):
            per.append(torch.randperm(Nk, generator=g)[:n_out].tolist())
        out.append(per)
    return out


def workload_prefill_inputs(w: Workload):
    return prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.N, w.d, w.dtype, w.seed, w.outlier_frac,
                          w.outlier_scale)


def decode_lengths(B, l_min, l_max, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(l_min, l_max + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def decode_inputs(B, Hq, Hkv, d, dtype="bf16", seed=0, l_min=1, l_max=512, max_len=None,
                  device="cpu", seq_lens=None):
    """Returns (seq_lens int32 [B] on CPU, q [B,Hq,d], k_cache, v_cache [B,Hkv,max_len,d]).

    q is on the CPU; the caches are on ``device``. Cache rows at positions >= L_b
    hold NaN. ``seq_lens`` may be given explicitly (then the length draw is
    still made, so q is the same as without it)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    drawn = torch.randint(l_min, l_max + 1, (B,), generator=g, dtype=torch.int64)
    lens = drawn.to(torch.int32) if seq_lens is None else torch.as_tensor(seq_lens,
                                                                          dtype=torch.int32)
    if max_len is None:
        max_len = l_max
    if int(lens.max()) > max_len or int(lens.min()) < 0:
        raise ValueError("sequence lengths must lie in [0, max_len]")
    t = DTYPES[dtype]
    q = torch.randn((B, Hq, d), generator=g, dtype=torch.float32).to(t)
    gd = torch.Generator(device=device).manual_seed(seed)
    kc = torch.full((B, Hkv, max_len, d), float("nan"), dtype=t, device=device)
    vc = torch.full((B, Hkv, max_len, d), float("nan"), dtype=t, device=device)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        kc[b, :, :L] = torch.randn((Hkv, L, d), generator=gd, dtype=torch.float32,
                                   device=device).to(t)
        vc[b, :, :L] = torch.randn((Hkv, L, d), generator=gd, dtype=torch.float32,
                                   device=device).to(t)
    return lens, q, kc, vc


def workload_decode_inputs(w: Workload, device="cpu"):
    return decode_inputs(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.seed, w.l_min, w.l_max,
                         max_len=w.l_max, device=device)


def bits(t: torch.Tensor):
    """Raw 16-bit patterns of a bf16/fp16 tensor as a numpy uint16 array (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def paged_from_padded(k_cache, v_cache, seq_lens, page_size, seed=0, spare=3):
    """Lays a padded cache [B,Hkv,max_len,d] out in a shuffled page pool.

    Returns (k_pages, v_pages [num_pages,page_size,Hkv,d], block_table [B,max_pages]
    int32 on the CPU). Sequence b's logical page p (rows p*page_size ..) goes to
    pool page block_table[b][p]; pages are assigned by a seeded permutation so
    neighbouring logical pages are scattered."""
    B, Hkv, max_len, d = k_cache.shape
    lens = [int(x) for x in torch.as_tensor(seq_lens)]
    max_pages = -(-max_len // page_size)
    need = [-(-L // page_size) for L in lens]
    num_pages = sum(need) + spare
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(num_pages, generator=g).tolist()
    dev = k_cache.device
    kp = torch.full((num_pages, page_size, Hkv, d), float("nan"), dtype=k_cache.dtype, device=dev)
    vp = torch.full_like(kp, float("nan"))
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        for p in range(need[b]):
            pg = perm[nxt]
            nxt += 1
            table[b, p] = pg
            r0, r1 = p * page_size, min(lens[b], (p + 1) * page_size)
            kp[pg, : r1 - r0] = k_cache[b, :, r0:r1].transpose(0, 1)
            vp[pg, : r1 - r0] = v_cache[b, :, r0:r1].transpose(0, 1)
    return kp, vp, table


def varlen_inputs(q_lens, k_lens, Hq, Hkv, d, dtype="bf16", seed=0):
    """Returns CPU tensors (q [total_q,Hq,d], k, v [total_k,Hkv,d], cu_q, cu_k [B+1] int32)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    cu_q = torch.zeros(len(q_lens) + 1, dtype=torch.int32)
    cu_k = torch.zeros(len(k_lens) + 1, dtype=torch.int32)
    cu_q[1:] = torch.cumsum(torch.as_tensor(q_lens, dtype=torch.int64), 0).to(torch.int32)
    cu_k[1:] = torch.cumsum(torch.as_tensor(k_lens, dtype=torch.int64), 0).to(torch.int32)
    t = DTYPES[dtype]
    q = torch.randn((int(cu_q[-1]), Hq, d), generator=g, dtype=torch.float32).to(t)
    k = torch.randn((int(cu_k[-1]), Hkv, d), generator=g, dtype=torch.float32).to(t)
    v = torch.randn((int(cu_k[-1]), Hkv, d), generator=g, dtype=torch.float32).to(t)
    return q, k, v, cu_q, cu_k


def varlen_lengths(total, n_min, n_max, seed):
    """Seeded sequence lengths, uniform on [n_min, n_max], until they fill `total`
    tokens (the last one is cut to fit)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    lens = []
    left = total
    while left > 0:
        n = int(torch.randint(n_min, n_max + 1, (1,), generator=g))
        lens.append(min(n, left))
        left -= lens[-1]
    return lens
