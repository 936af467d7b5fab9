"""attn_bwd_noalloc (the backward with D in the library's fixed scratch, for
callers that cannot allocate) against attn_bwd (D in a caller buffer), through
the C ABI: two calls in a row on one GPU, the first at the scratch's maximum
size (B * Hq * Nq = 2^22 rows), the second smaller, each bit-identical to
attn_bwd on the same inputs (same kernels, same arithmetic), and the small one
also against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import exact_attention_46_amd as ea
import oracle
from grad_bound import grad_bound
from exact_attention_46_amd import workloads as wl

pytestmark = pytest.mark.gpu

SCRATCH_ROWS = 1 << 22


def _inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    t = wl.DTYPES[dtype]
    q = torch.randn((B, Hq, Nq, d), generator=g, device="cuda").to(t)
    k = torch.randn((B, Hkv, Nk, d), generator=g, device="cuda").to(t)
    v = torch.randn((B, Hkv, Nk, d), generator=g, device="cuda").to(t)
    do = torch.randn((B, Hq, Nq, d), generator=g, device="cuda").to(t)
    return q, k, v, do


def _both(q, k, v, do, causal, scale):
    o, lse = ea.fwd(q, k, v, causal=causal, scale=scale)
    ref = ea.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    ea.attn_bwd_noalloc(q, k, v, o, do, lse, got[0], got[1], got[2], causal, scale)
    torch.cuda.synchronize()
    return ref, got


def test_bwd_noalloc_matches_bwd_two_calls():
    # call 1: the largest problem the scratch holds (2^22 query rows; Nq > Nk,
    # so the first Nq - Nk rows of every head see no key: dq = 0 there)
    B, Hq, Hkv, Nq, Nk, d = 1, 32, 8, 1 << 17, 256, 128
    assert B * Hq * Nq == SCRATCH_ROWS
    q, k, v, do = _inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", 11)
    ref, got = _both(q, k, v, do, True, 1.0 / math.sqrt(d))
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "call 1: %s differs" % name
    assert not got[0][:, :, : Nq - Nk].any(), "rows with no key must get dq = 0"
    del q, k, v, do, ref, got
    torch.cuda.empty_cache()
    # call 2: smaller, another dtype, d and mask, right after (the scratch keeps
    # call 1's values where call 2 does not write; call 2 must not read them)
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 300, 300, 64
    q, k, v, do = _inputs(B, Hq, Hkv, Nq, Nk, d, "fp16", 12)
    scale = 1.0 / math.sqrt(d)
    ref, got = _both(q, k, v, do, False, scale)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "call 2: %s differs" % name
    rq, rk, rv = oracle.attn_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do), 1, scale, False)
    bounds = grad_bound(q, k, v, do, "fp16", scale, False)
    for name, g, r, bnd in zip(("dq", "dk", "dv"), got, (rq, rk, rv), bounds):
        gv = g.float().cpu().double().numpy()
        err = np.abs(gv - r)
        assert (err <= bnd).all(), "call 2: %s vs oracle: error/bound %.3f" % (
            name, float((err / np.maximum(bnd, 1e-300)).max()))


def test_bwd_noalloc_rejects_more_rows_than_the_scratch():
    q = torch.zeros((1, 33, 1 << 17, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 33, 1 << 17), dtype=torch.float32, device="cuda")
    with pytest.raises(ea.AttnError) as e:
        ea.attn_bwd_noalloc(q, k, k, q, q, lse, q, k, k, True, 0.1)
    assert e.value.status == ea._binding.ERR_SCRATCH
