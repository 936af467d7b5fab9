"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerances (on the same seeded inputs): max |O_gpu - O_ref| <= 1e-2 for bf16 and
<= 4e-3 for fp16, max |LSE_gpu - LSE_ref| <= 1e-3, -inf LSE exactly where the
oracle has it, and no NaN / Inf anywhere in O. Outputs are written into buffers
with guard bands that must come back untouched.

Small shapes are compared element by element (they span several tiles and a
ragged tail); the full-size workloads are compared on seeded samples of rows
that the oracle computes one by one, plus whole-tensor properties.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import exact_attention_46_amd as ea
import oracle
from exact_attention_46_amd import workloads as wl
from grad_bound import grad_bound

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 1e-2, "fp16": 4e-3}
TOL_LSE = 1e-3
GUARD = 256  # elements of guard band on each side of an output buffer
SENTINEL_F32 = 12345.678


def _guarded(shape, dtype, dev="cuda"):
    n = int(np.prod(shape))
    if dtype == torch.float32:
        buf = torch.full((n + 2 * GUARD,), SENTINEL_F32, dtype=dtype, device=dev)
    else:
        buf = torch.full((n + 2 * GUARD,), 0, dtype=torch.int16, device=dev)
        buf.fill_(0x5A5A)
        buf = buf.view(dtype)
    return buf, buf[GUARD:GUARD + n].view(shape)


def _guard_ok(buf, n):
    b = buf.detach().cpu()
    if b.dtype == torch.float32:
        ok = (b[:GUARD] == SENTINEL_F32).all() and (b[GUARD + n:] == SENTINEL_F32).all()
    else:
        bi = b.view(torch.int16)
        ok = (bi[:GUARD] == 0x5A5A).all() and (bi[GUARD + n:] == 0x5A5A).all()
    return bool(ok)


def _report(err, ref):
    i = np.unravel_index(np.argmax(err), err.shape)
    return "max err %.3e at %s (|ref| there %.3f)" % (err[i], i, abs(ref[i]))


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what, floor_aware=False):
    o = o_gpu.detach().float().cpu().double().numpy()
    lse = lse_gpu.detach().cpu().double().numpy()
    assert np.isfinite(o).all(), "%s: NaN/Inf in O" % what
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), "%s: -inf LSE mismatch" % what
    assert not np.isnan(lse).any(), "%s: NaN in LSE" % what
    err = np.abs(o - o_ref)
    if floor_aware:
        # bf16 output rounding alone can exceed the gate; judge the excess over it
        t = wl.DTYPES[dtype]
        floor = np.abs(torch.from_numpy(o_ref).to(t).double().numpy() - o_ref)
        gate = err - floor
        assert gate.max() <= TOL_O[dtype], "%s: O excess over rounding floor: %s" % (
            what, _report(gate, o_ref))
    else:
        assert err.max() <= TOL_O[dtype], "%s: O %s" % (what, _report(err, o_ref))
    fin = np.isfinite(lse_ref)
    if fin.any():
        lerr = np.abs(lse[fin] - lse_ref[fin])
        assert lerr.max() <= TOL_LSE, "%s: LSE max err %.3e" % (what, lerr.max())
    return err.max()


def run_fwd(q, k, v, causal, scale):
    B, Hq, Nq, d = q.shape
    ob, o = _guarded(q.shape, q.dtype)
    lb, lse = _guarded((B, Hq, Nq), torch.float32)
    ea.attn_fwd(q, k, v, o, lse, causal, scale)
    torch.cuda.synchronize()
    assert _guard_ok(ob, o.numel()) and _guard_ok(lb, lse.numel()), "write outside the outputs"
    return o, lse


def _dev(*ts):
    return [t.cuda() for t in ts]


# --------------------------------------------------------------- prefill, full compare

def test_tiny_workload_both_masks():
    w = wl.WORKLOADS["tiny"]
    q, k, v = wl.workload_prefill_inputs(w)
    for causal in (False, True):
        o, lse = run_fwd(*_dev(q, k, v), causal, w.scale)
        ro, rl = oracle.attn_fwd(wl.bits(q), wl.bits(k), wl.bits(v), 1, w.scale, causal)
        check(o, lse, ro, rl, "fp16", "tiny causal=%d" % causal)


EDGE = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, causal
    (1, 2, 2, 1, 1, 128, "bf16", True),
    (1, 2, 2, 17, 17, 64, "fp16", True),
    (2, 4, 1, 64, 64, 128, "bf16", False),
    (1, 8, 2, 127, 127, 128, "bf16", True),
    (1, 4, 4, 128, 128, 64, "bf16", True),
    (1, 4, 4, 129, 129, 128, "fp16", True),
    (1, 8, 1, 1000, 1000, 128, "bf16", True),
    (1, 8, 8, 1000, 1000, 64, "fp16", False),
    (1, 4, 2, 100, 300, 128, "bf16", True),
    (1, 4, 2, 300, 100, 128, "bf16", True),
    (1, 4, 2, 300, 100, 64, "fp16", False),
    (1, 2, 2, 1, 513, 128, "bf16", True),
    (1, 2, 2, 513, 1, 64, "fp16", False),
    (2, 8, 8, 257, 257, 128, "bf16", False),
    (1, 32, 8, 300, 300, 128, "bf16", True),
    (3, 6, 3, 70, 200, 128, "fp16", True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal", EDGE)
def test_fwd_edge_shapes(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    seed = zlib.crc32(repr((B, Hq, Hkv, Nq, Nk, d, dtype, causal)).encode()) % 10000
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fwd(*_dev(q, k, v), causal, scale)
    ro, rl = oracle.attn_fwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.DTYPE_CODE[dtype], scale,
                             causal)
    check(o, lse, ro, rl, dtype, "edge %s" % ((B, Hq, Hkv, Nq, Nk, d, dtype, causal),))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fwd_score_outliers_exercise_rescale(dtype):
    # 1% of key rows x10 (the long-context stress pattern) at a size the oracle
    # finishes whole: rows jump in max many times. Rows are then nearly one-hot
    # and |O| exceeds 4, where bf16 rounding alone exceeds 1e-2, so the bf16 run
    # is judged on the excess over that rounding; the fp16 run (half an ulp is
    # 2^-9 there) takes the plain 4e-3 gate.
    B, H, N, d = 1, 4, 2048, 128
    q, k, v = wl.prefill_inputs(B, H, H, N, N, d, dtype, 44, outlier_frac=0.01,
                                outlier_scale=10.0)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fwd(*_dev(q, k, v), True, scale)
    ro, rl = oracle.attn_fwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.DTYPE_CODE[dtype], scale,
                             True)
    check(o, lse, ro, rl, dtype, "outliers", floor_aware=(dtype == "bf16"))


def test_fwd_nan_only_poisons_rows_that_see_it():
    B, H, N, d = 1, 2, 200, 128
    q, k, v = wl.prefill_inputs(B, H, H, N, N, d, "bf16", 55)
    k[0, 0, 150, 3] = float("nan")  # key 150 of head 0
    o, lse = run_fwd(*_dev(q, k, v), True, 1.0 / math.sqrt(d))
    o = o.float().cpu()
    assert torch.isfinite(o[0, 0, :150]).all()
    assert torch.isnan(o[0, 0, 150:]).all()
    assert torch.isfinite(o[0, 1]).all()


# Non-finite inputs (a NaN or Inf must reach exactly the rows that attend to its
# key). Plants: (tensor, batch, head, key row, column, value); keys placed in
# tiles the causal or window limits cut through, so some rows of the same tile
# must not see them.
NONFINITE = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, mask (True causal, False none, (left, right)), plants
    (1, 4, 2, 300, 300, 128, "bf16", True,
     [("v", 0, 0, 150, 3, "nan"), ("v", 0, 0, 170, 5, "inf"), ("v", 0, 1, 10, 0, "-inf"),
      ("k", 0, 1, 200, 7, "nan"), ("v", 0, 1, 40, 9, "inf")]),
    (1, 2, 2, 200, 300, 64, "fp16", True,
     [("v", 0, 0, 250, 1, "inf"), ("k", 0, 1, 180, 2, "inf"), ("v", 0, 1, 299, 0, "nan")]),
    (1, 2, 2, 300, 300, 128, "bf16", False,
     [("v", 0, 0, 77, 4, "nan"), ("k", 0, 1, 130, 0, "nan")]),
    (1, 2, 2, 300, 300, 128, "bf16", (50, 0),
     [("v", 0, 0, 100, 6, "nan"), ("v", 0, 1, 260, 2, "-inf"), ("k", 0, 1, 40, 1, "nan")]),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,mask,plants", NONFINITE)
def test_fwd_nonfinite_reaches_only_attending_rows(B, Hq, Hkv, Nq, Nk, d, dtype, mask, plants):
    seed = zlib.crc32(repr(("nonfinite", B, Hq, Hkv, Nq, Nk, d, dtype)).encode()) % 10000
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed)
    for name, b, h, j, c, val in plants:
        {"k": k, "v": v}[name][b, h, j, c] = float(val)
    scale = 1.0 / math.sqrt(d)
    dc = wl.DTYPE_CODE[dtype]
    qd, kd, vd = _dev(q, k, v)
    if isinstance(mask, tuple):
        o = torch.empty_like(qd)
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
        ea.attn_fwd_local(qd, kd, vd, o, lse, mask[0], mask[1], scale)
        torch.cuda.synchronize()
        ro, rl = oracle.attn_fwd_local(wl.bits(q), wl.bits(k), wl.bits(v), dc, scale, *mask)
    else:
        o, lse = run_fwd(qd, kd, vd, mask, scale)
        ro, rl = oracle.attn_fwd(wl.bits(q), wl.bits(k), wl.bits(v), dc, scale, mask)
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    what = "non-finite %s" % ((B, Hq, Hkv, Nq, Nk, d, dtype, mask),)
    # the same elements are NaN, +Inf and -Inf as in the oracle's exact result
    for f in (np.isnan, np.isposinf, np.isneginf):
        bad = np.argwhere(f(og) != f(ro))
        assert bad.size == 0, "%s: %s differs at %d elements, first %s (gpu %r, oracle %r)" % (
            what, f.__name__, len(bad), tuple(bad[0]), og[tuple(bad[0])], ro[tuple(bad[0])])
    assert np.array_equal(np.isnan(lg), np.isnan(rl)), what + ": NaN LSE pattern"
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl)), what + ": -inf LSE pattern"
    assert (~np.isfinite(ro)).any(), what + ": nothing planted reached an output"
    fin = np.isfinite(ro)
    assert fin.any(), what + ": no finite output left to compare"
    assert np.abs(og[fin] - ro[fin]).max() <= TOL_O[dtype], what + ": finite O"
    lfin = np.isfinite(rl)
    if lfin.any():
        assert np.abs(lg[lfin] - rl[lfin]).max() <= TOL_LSE, what + ": finite LSE"


# --------------------------------------------------------------- prefill, full size

def _sample_rows(B, H, N, per_unit, seed, extra=(), extra_per_head=None):
    """Seeded rows per (b, h): `per_unit` drawn without replacement, plus `extra`
    (every unit) and `extra_per_head(b, h)` (that unit)."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        for h in range(H):
            picks = set(rng.choice(N, size=min(per_unit, N), replace=False).tolist())
            picks.update([0, N - 1])
            picks.update(extra)
            if extra_per_head is not None:
                picks.update(extra_per_head(b, h))
            rows += [(b, h, i) for i in sorted(picks) if 0 <= i < N]
    return np.array(rows, dtype=np.int64)


def _full_size(name, rows_of, floor_aware=False):
    w = wl.WORKLOADS[name]
    q, k, v = wl.workload_prefill_inputs(w)
    o, lse = run_fwd(*_dev(q, k, v), True, w.scale)
    # whole-tensor properties
    assert torch.isfinite(o).all()
    assert torch.isfinite(lse).all()
    rows = rows_of(w)
    ro, rl = oracle.attn_fwd_rows(wl.bits(q), wl.bits(k), wl.bits(v), 0, w.scale, True, rows)
    idx = torch.from_numpy(rows)
    og = o.cpu()[idx[:, 0], idx[:, 1], idx[:, 2]]
    lg = lse.cpu()[idx[:, 0], idx[:, 1], idx[:, 2]]
    print("%s: %d rows compared" % (name, len(rows)))
    return check(og, lg, ro, rl, w.dtype, name, floor_aware=floor_aware)


def _edges(N):
    return list(range(64)) + list(range(N - 64, N))


def test_llm_prefill_full_size_every_row():
    """The whole llm_prefill workload (B=4, H=32, N=2048) in the launch the
    benchmark times, every one of its 262 144 rows against the oracle."""
    w = wl.WORKLOADS["llm_prefill"]
    q, k, v = wl.workload_prefill_inputs(w)
    o, lse = run_fwd(*_dev(q, k, v), True, w.scale)
    ro, rl = oracle.attn_fwd(wl.bits(q), wl.bits(k), wl.bits(v), 0, w.scale, True)
    check(o, lse, ro, rl, w.dtype, "llm_prefill, every row")


def test_gqa_prefill_full_size_sampled():
    """256 seeded rows of every (b, h) plus its first and last 64 rows."""
    _full_size("gqa_prefill",
               lambda w: _sample_rows(w.B, w.Hq, w.N, 256, w.seed, extra=_edges(w.N)))


def test_long_context_full_size_sampled():
    """256 seeded rows of every head plus its first and last 64 rows, plus every
    query row at the index of one of the head's outlier (x10) keys; the gate is
    on the excess over the bf16 rounding of the exact result (outputs reach
    |O| > 4 there, where that rounding alone exceeds 1e-2)."""
    w = wl.WORKLOADS["long_context"]
    outl = wl.outlier_rows(w.B, w.Hq, w.Hkv, w.N, w.N, w.d, w.seed, w.outlier_frac)
    group = w.Hq // w.Hkv
    _full_size("long_context",
               lambda w: _sample_rows(w.B, w.Hq, w.N, 256, w.seed, extra=_edges(w.N),
                                      extra_per_head=lambda b, h: outl[b][h // group]),
               floor_aware=True)


# --------------------------------------------------------------- decode

# 64 sequence lengths (max_len 1024) that give 8 840 items at 32-key chunks and
# 8 kv-heads, at least eight per wave on a 256-CU device: the split kernel then
# takes the full chunks first and the short last chunks after them, longest
# first. They include 0, exact multiples of the chunk (no short chunk), a short
# chunk alone (8) and equal remainders (1000, 1000, 1000 and 8 all leave 8 keys).
ORDERED_LENS = [(37 * i * i + 11 * i) % 1025 for i in range(64)]
for _i, _L in {0: 0, 1: 1024, 2: 64, 3: 1000, 4: 1000, 5: 8, 6: 40, 7: 72, 8: 1023, 9: 1000,
               24: 1024, 31: 1024}.items():
    ORDERED_LENS[_i] = _L

DECODE = [
    # B, Hq, Hkv, d, dtype, lens, max_len, chunk
    (5, 8, 2, 128, "bf16", [1, 9, 0, 31, 16], 32, 16),
    (4, 32, 8, 128, "bf16", None, 2048, 512),
    (3, 4, 4, 64, "fp16", [700, 1, 513], 1024, 64),
    (2, 32, 1, 128, "bf16", [1500, 333], 1536, 100),
    (6, 16, 2, 64, "bf16", [5, 40, 77, 128, 129, 3], 130, 7),
    (2, 8, 8, 128, "fp16", [4096, 4000], 4096, 4096),
    # 16 384 / 12 288 items for 1 024 waves: every wave walks many items that are
    # a single 32-key tile (chunk 32) or one tile and a 16-key tail (chunk 48),
    # so an item's Q rows are fetched right after the previous item's stores
    (64, 32, 8, 128, "bf16", None, 1024, 32),
    (64, 32, 8, 128, "bf16", None, 1024, 48),
    (64, 16, 8, 64, "fp16", None, 1024, 32),
    # 8 840 items, at least eight per wave on a 256-CU device (see ORDERED_LENS)
    (64, 32, 8, 128, "bf16", ORDERED_LENS, 1024, 32),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,dtype,lens,max_len,chunk", DECODE)
def test_decode_split_and_combine(B, Hq, Hkv, d, dtype, lens, max_len, chunk):
    seed = 1000 + B * 7 + Hq + d
    sl, q, kc, vc = wl.decode_inputs(B, Hq, Hkv, d, dtype, seed, l_min=1, l_max=max_len,
                                     max_len=max_len, device="cpu", seq_lens=lens)
    scale = 1.0 / math.sqrt(d)
    qd, kcd, vcd, sld = _dev(q, kc, vc, sl)
    C = -(-max_len // chunk)
    pob, po = _guarded((B, Hq, C, d), torch.float32)
    plb, pl = _guarded((B, Hq, C), torch.float32)
    ob, o = _guarded((B, Hq, d), q.dtype)
    lb, lse = _guarded((B, Hq), torch.float32)
    ea.attn_decode_split(qd, kcd, vcd, sld, po, pl, chunk, scale)
    ea.attn_decode_combine(po, pl, sld, o, lse, chunk)
    torch.cuda.synchronize()
    for buf, t in ((pob, po), (plb, pl), (ob, o), (lb, lse)):
        assert _guard_ok(buf, t.numel()), "write outside an output"
    dc = wl.DTYPE_CODE[dtype]
    # partials, chunk by chunk (slots past the end only need LSE = -inf)
    rpo, rpl = oracle.decode_chunks(wl.bits(q), wl.bits(kc), wl.bits(vc), sl.numpy(), dc, chunk,
                                    scale)
    pl_h = pl.cpu().double().numpy()
    assert np.array_equal(np.isneginf(pl_h), np.isneginf(rpl))
    valid = np.isfinite(rpl)
    po_h = po.cpu().double().numpy()
    assert np.isfinite(po_h[valid]).all()
    assert np.abs(po_h[valid] - rpo[valid]).max() <= TOL_O[dtype]
    assert np.abs(pl_h[valid] - rpl[valid]).max() <= TOL_LSE
    # final output against the direct decode
    ro, rl = oracle.decode(wl.bits(q), wl.bits(kc), wl.bits(vc), sl.numpy(), dc, scale)
    check(o, lse, ro, rl, dtype, "decode")
    # the GPU combine against the oracle's combine of the very same partials
    co, cl = oracle.combine(po_h, pl_h, sl.numpy(), chunk)
    check(o, lse, co, cl, dtype, "combine of GPU partials")


def test_decode_combine_alone_with_empty_chunks():
    B, Hq, C, d, chunk = 3, 4, 6, 128, 10
    g = torch.Generator().manual_seed(7)
    po = torch.randn((B, Hq, C, d), generator=g)
    pl = torch.randn((B, Hq, C), generator=g) * 5
    pl[0, 1, 2] = float("-inf")
    pl[1, :, :] = float("-inf")  # every chunk empty
    sl = torch.tensor([60, 25, 1], dtype=torch.int32)
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ea.attn_decode_combine(po.cuda(), pl.cuda(), sl.cuda(), o, lse, chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.combine(po.double().numpy(), pl.double().numpy(), sl.numpy(), chunk)
    check(o, lse, ro, rl, "bf16", "combine alone")
    assert (o[1].float() == 0).all()


def test_decode_full_size_every_sequence():
    """The decode workload (64 sequences, L ~ U[512, 32768], 512-key chunks) in
    the launches the benchmark times: every valid chunk partial of every
    sequence against the oracle's chunk partials, and every final output
    against the oracle's direct decode."""
    w = wl.WORKLOADS["decode"]
    sl, q, kc, vc = wl.workload_decode_inputs(w, device="cuda")
    qd, sld = q.cuda(), sl.cuda()
    C = -(-w.l_max // w.chunk)
    pob, po = _guarded((w.B, w.Hq, C, w.d), torch.float32)
    plb, pl = _guarded((w.B, w.Hq, C), torch.float32)
    ob, o = _guarded((w.B, w.Hq, w.d), torch.bfloat16)
    lb, lse = _guarded((w.B, w.Hq), torch.float32)
    ea.attn_decode_split(qd, kc, vc, sld, po, pl, w.chunk, w.scale)
    ea.attn_decode_combine(po, pl, sld, o, lse, w.chunk)
    torch.cuda.synchronize()
    for buf, t in ((pob, po), (plb, pl), (ob, o), (lb, lse)):
        assert _guard_ok(buf, t.numel()), "write outside an output"
    kb, vb = wl.bits(kc), wl.bits(vc)  # rows past each length are NaN and never read
    lens = sl.numpy()
    rpo, rpl = oracle.decode_chunks(wl.bits(q), kb, vb, lens, 0, w.chunk, w.scale)
    pl_h = pl.cpu().double().numpy()
    assert np.array_equal(np.isneginf(pl_h), np.isneginf(rpl))
    valid = np.isfinite(rpl)
    assert valid.sum() == w.Hq * int(sum(-(-int(L) // w.chunk) for L in lens))
    po_h = po.cpu().double().numpy()
    assert np.isfinite(po_h[valid]).all()
    perr = np.abs(po_h[valid] - rpo[valid]).max()
    assert perr <= TOL_O["bf16"], "partials: O max err %.3e" % perr
    assert np.abs(pl_h[valid] - rpl[valid]).max() <= TOL_LSE
    ro, rl = oracle.decode(wl.bits(q), kb, vb, lens, 0, w.scale)
    check(o, lse, ro, rl, "bf16", "decode, every sequence")


# --------------------------------------------------------------- decode, combine fused

FUSED = [
    # B, Hq, Hkv, d, dtype, lens, max_len, chunk
    (5, 8, 2, 128, "bf16", [1, 9, 0, 31, 16], 32, 16),        # empty and one-chunk sequences
    (4, 32, 8, 128, "bf16", None, 2048, 512),
    (3, 4, 4, 64, "fp16", [700, 1, 513], 1024, 64),
    (2, 32, 1, 128, "bf16", [1500, 333], 1536, 100),          # 32 heads per kv-head, ragged chunks
    (6, 16, 2, 64, "bf16", [5, 40, 77, 128, 129, 3], 130, 7),
    (64, 32, 8, 128, "bf16", None, 1024, 32),                 # many one-tile items per wave
    (16, 8, 8, 128, "bf16", None, 4096, 64),                  # up to 64 chunks per pair
    (2, 8, 8, 128, "fp16", [4096, 4000], 4096, 4096),         # every sequence one chunk
    (64, 32, 8, 128, "bf16", ORDERED_LENS, 1024, 32),         # full chunks first, then short
]


def _fused_call(q, kc, vc, sl, ws, chunk, scale):
    B, Hq, d = q.shape
    ob, o = _guarded((B, Hq, d), q.dtype)
    lb, lse = _guarded((B, Hq), torch.float32)
    ea.attn_decode_fused(q, kc, vc, sl, o, lse, ws, chunk, scale)
    torch.cuda.synchronize()
    assert _guard_ok(ob, o.numel()) and _guard_ok(lb, lse.numel()), "write outside an output"
    return o, lse


@pytest.mark.parametrize("B,Hq,Hkv,d,dtype,lens,max_len,chunk", FUSED)
def test_decode_fused(B, Hq, Hkv, d, dtype, lens, max_len, chunk):
    """The combine fused into the split kernel (last chunk of each (sequence,
    kv-head) merges): against the oracle's direct decode and against the
    two-kernel split + combine at the same chunk, twice on one workspace (the
    kernel resets its counters), the second call on other lengths."""
    seed = 4000 + B * 7 + Hq + d + chunk
    sl, q, kc, vc = wl.decode_inputs(B, Hq, Hkv, d, dtype, seed, l_min=1, l_max=max_len,
                                     max_len=max_len, device="cpu", seq_lens=lens)
    scale = 1.0 / math.sqrt(d)
    dc = wl.DTYPE_CODE[dtype]
    qd, kcd, vcd, sld = _dev(q, kc, vc, sl)
    n = ea.attn_decode_fused_workspace(B, Hq, Hkv, max_len, d, chunk)
    wsb, ws = _guarded((n,), torch.float32)  # the guard band keeps 256-byte alignment
    ws.zero_()
    for call in range(2):
        if call == 1:  # shorter lengths (rows past the first lengths are NaN), one empty
            g = torch.Generator().manual_seed(seed + 1)
            sl = torch.minimum(torch.randint(0, max_len + 1, (B,), generator=g,
                                             dtype=torch.int32), sl)
            sl[0] = 0
            sld = sl.cuda()
        o, lse = _fused_call(qd, kcd, vcd, sld, ws, chunk, scale)
        counters = ws[:B * Hkv].view(torch.int32).cpu()
        assert (counters == 0).all(), "counters not reset: %s" % counters[counters != 0][:8]
        ro, rl = oracle.decode(wl.bits(q), wl.bits(kc), wl.bits(vc), sl.numpy(), dc, scale)
        check(o, lse, ro, rl, dtype, "fused decode, call %d" % call,
              floor_aware=max_len <= 64)
        # against the two-kernel path at the same chunk
        o2, l2 = ea.decode(qd, kcd, vcd, sld, chunk=chunk, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(torch.isneginf(lse), torch.isneginf(l2))
        fin = torch.isfinite(l2)
        assert (lse[fin] - l2[fin]).abs().max().item() <= 1e-5
        assert (o.float() - o2.float()).abs().max().item() <= TOL_O[dtype] / 2
    assert _guard_ok(wsb, ws.numel()), "write outside the workspace"


def test_decode_fused_full_size_every_sequence():
    """The fused decode on the whole decode workload (64 sequences, 512-key
    chunks, up to 64 chunks per pair): every sequence against the oracle."""
    w = wl.WORKLOADS["decode"]
    sl, q, kc, vc = wl.workload_decode_inputs(w, device="cuda")
    qd, sld = q.cuda(), sl.cuda()
    ws = ea.fused_workspace(w.B, w.Hq, w.Hkv, w.l_max, w.d, w.chunk)
    for call in range(2):  # the second call reuses the workspace the first reset
        o, lse = ea.decode_fused(qd, kc, vc, sld, chunk=w.chunk, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert (ws[:w.B * w.Hkv].view(torch.int32) == 0).all()
    ro, rl = oracle.decode(wl.bits(q), wl.bits(kc), wl.bits(vc), sl.numpy(), 0, w.scale)
    check(o, lse, ro, rl, "bf16", "fused decode, every sequence")
    # the paged cache through the fused path: bit-identical to the contiguous one
    kp, vp, table = wl.paged_from_padded(kc, vc, sl, 64, seed=w.seed)
    o_p = torch.empty_like(o)
    l_p = torch.empty_like(lse)
    ea.attn_decode_fused_paged(qd, kp, vp, table.cuda(), sld, o_p, l_p, ws, w.chunk, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o.view(torch.int16))
    assert torch.equal(l_p, lse)


@pytest.mark.parametrize("B,Hq,Hkv,d,dtype,lens,max_len,page_size,chunk", [
    (5, 8, 2, 128, "bf16", [1, 9, 0, 31, 16], 32, 16, 32),
    (3, 4, 4, 64, "fp16", [700, 1, 513], 1024, 64, 64),
    (6, 16, 2, 64, "bf16", [5, 40, 77, 128, 129, 3], 160, 32, 48),
    (64, 32, 8, 128, "bf16", None, 1024, 32, 32),
])
def test_paged_decode_fused(B, Hq, Hkv, d, dtype, lens, max_len, page_size, chunk):
    seed = 5000 + B * 7 + Hq + d + page_size
    sl, q, kc, vc = wl.decode_inputs(B, Hq, Hkv, d, dtype, seed, l_min=1, l_max=max_len,
                                     max_len=max_len, device="cpu", seq_lens=lens)
    kp, vp, table = wl.paged_from_padded(kc, vc, sl, page_size, seed=seed)
    scale = 1.0 / math.sqrt(d)
    qd, kpd, vpd, td, sld = _dev(q, kp, vp, table, sl)
    max_pages = table.shape[1]
    ws = ea.fused_workspace(B, Hq, Hkv, max_pages * page_size, d, chunk)
    ob, o = _guarded((B, Hq, d), q.dtype)
    lb, lse = _guarded((B, Hq), torch.float32)
    ea.attn_decode_fused_paged(qd, kpd, vpd, td, sld, o, lse, ws, chunk, scale)
    torch.cuda.synchronize()
    assert _guard_ok(ob, o.numel()) and _guard_ok(lb, lse.numel()), "write outside an output"
    assert (ws[:B * Hkv].view(torch.int32) == 0).all()
    ro, rl = oracle.decode_paged(wl.bits(q), wl.bits(kp), wl.bits(vp), table.numpy(),
                                 sl.numpy(), wl.DTYPE_CODE[dtype], scale)
    check(o, lse, ro, rl, dtype, "paged fused decode", floor_aware=max_len <= 64)


# --------------------------------------------------------------- paged decode

PAGED = [
    # B, Hq, Hkv, d, dtype, lens, max_len, page_size, chunk
    (5, 8, 2, 128, "bf16", [1, 9, 0, 31, 16], 32, 16, 32),
    (4, 32, 8, 128, "bf16", None, 2048, 128, 512),
    (3, 4, 4, 64, "fp16", [700, 1, 513], 1024, 64, 64),
    (2, 32, 1, 128, "bf16", [1500, 333], 1536, 48, 96),
    (6, 16, 2, 64, "bf16", [5, 40, 77, 128, 129, 3], 160, 32, 48),
    (3, 8, 2, 128, "bf16", [700, 256, 17], 768, 16, 256),
    (2, 8, 8, 128, "fp16", [4096, 4000], 4096, 512, 4096),
    # many single-tile items per wave (see DECODE)
    (64, 32, 8, 128, "bf16", None, 1024, 32, 32),
    # full chunks first, then the short ones (see ORDERED_LENS)
    (64, 32, 8, 128, "bf16", ORDERED_LENS, 1024, 32, 32),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,dtype,lens,max_len,page_size,chunk", PAGED)
def test_paged_decode_split_and_combine(B, Hq, Hkv, d, dtype, lens, max_len, page_size, chunk):
    seed = 2000 + B * 7 + Hq + d + page_size
    sl, q, kc, vc = wl.decode_inputs(B, Hq, Hkv, d, dtype, seed, l_min=1, l_max=max_len,
                                     max_len=max_len, device="cpu", seq_lens=lens)
    kp, vp, table = wl.paged_from_padded(kc, vc, sl, page_size, seed=seed)
    scale = 1.0 / math.sqrt(d)
    qd, kpd, vpd, td, sld = _dev(q, kp, vp, table, sl)
    max_pages = table.shape[1]
    C = -(-(max_pages * page_size) // chunk)
    pob, po = _guarded((B, Hq, C, d), torch.float32)
    plb, pl = _guarded((B, Hq, C), torch.float32)
    ob, o = _guarded((B, Hq, d), q.dtype)
    lb, lse = _guarded((B, Hq), torch.float32)
    ea.attn_decode_split_paged(qd, kpd, vpd, td, sld, po, pl, chunk, scale)
    ea.attn_decode_combine(po, pl, sld, o, lse, chunk)
    torch.cuda.synchronize()
    for buf, t in ((pob, po), (plb, pl), (ob, o), (lb, lse)):
        assert _guard_ok(buf, t.numel()), "write outside an output"
    dc = wl.DTYPE_CODE[dtype]
    ro, rl = oracle.decode_paged(wl.bits(q), wl.bits(kp), wl.bits(vp), table.numpy(),
                                 sl.numpy(), dc, scale)
    check(o, lse, ro, rl, dtype, "paged decode")
    pl_h = pl.cpu().double().numpy()
    lens_h = sl.numpy()
    for b in range(B):  # chunk slots past the end of a sequence carry LSE = -inf
        nc = -(-int(lens_h[b]) // chunk)
        assert np.isneginf(pl_h[b, :, nc:]).all() and np.isfinite(pl_h[b, :, :nc]).all()


def test_paged_decode_rejects_unsupported_geometry():
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((4, 24, 2, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    sl = torch.ones((1,), dtype=torch.int32, device="cuda")
    po = torch.empty((1, 4, 1, 128), dtype=torch.float32, device="cuda")
    pl = torch.empty((1, 4, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(ea.AttnError):  # page size 24 is not a multiple of 16
        ea.attn_decode_split_paged(q, kp, kp, table, sl, po, pl, 48, 0.1)


def test_paged_decode_full_size_matches_contiguous_and_oracle():
    """The decode workload laid out in 64-row pages: bit-identical to the
    contiguous split kernel (same tiles, same arithmetic), and sampled
    sequences against the oracle."""
    w = wl.WORKLOADS["decode"]
    sl, q, kc, vc = wl.workload_decode_inputs(w, device="cuda")
    kp, vp, table = wl.paged_from_padded(kc, vc, sl, 64, seed=w.seed)
    qd, sld, td = q.cuda(), sl.cuda(), table.cuda()
    o_p, lse_p = ea.decode_paged(qd, kp, vp, td, sld, chunk=w.chunk, scale=w.scale)
    o_c, lse_c = ea.decode(qd, kc, vc, sld, chunk=w.chunk, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o_c.view(torch.int16))
    assert torch.equal(lse_p, lse_c)
    lens = sl.numpy()
    for b in sorted({int(np.argmax(lens)), int(np.argmin(lens)), 5, 38}):
        L = int(lens[b])
        ro, rl = oracle.decode(wl.bits(q[b:b + 1]), wl.bits(kc[b:b + 1, :, :L].cpu()),
                               wl.bits(vc[b:b + 1, :, :L].cpu()), np.array([L], dtype=np.int32),
                               0, w.scale)
        check(o_p[b:b + 1], lse_p[b:b + 1], ro, rl, "bf16", "paged decode seq %d (L=%d)" % (b, L))


# --------------------------------------------------------------- packed variable-length prefill

VARLEN = [
    # q_lens, k_lens, Hq, Hkv, d, dtype, causal
    ([1, 255, 256, 257, 0, 600], [1, 255, 256, 257, 0, 600], 4, 2, 128, "bf16", True),
    ([300, 5, 1000], [500, 5, 1000], 8, 8, 64, "fp16", True),
    ([700, 64, 3], [100, 0, 3], 4, 1, 128, "bf16", True),
    ([129, 513, 2], [129, 513, 2], 6, 3, 128, "bf16", False),
    ([2048, 1536, 100], [2048, 1536, 100], 32, 8, 128, "bf16", True),
]


@pytest.mark.parametrize("q_lens,k_lens,Hq,Hkv,d,dtype,causal", VARLEN)
def test_fwd_varlen(q_lens, k_lens, Hq, Hkv, d, dtype, causal):
    seed = zlib.crc32(repr((q_lens, k_lens, Hq, d)).encode()) % 10000
    q, k, v, cq, ck = wl.varlen_inputs(q_lens, k_lens, Hq, Hkv, d, dtype, seed)
    scale = 1.0 / math.sqrt(d)
    total_q = q.shape[0]
    ob, o = _guarded(q.shape, q.dtype)
    lb, lse = _guarded((Hq, total_q), torch.float32)
    qd, kd, vd, cqd, ckd = _dev(q, k, v, cq, ck)
    ea.attn_fwd_varlen(qd, kd, vd, o, lse, cqd, ckd, max(q_lens), causal, scale)
    torch.cuda.synchronize()
    assert _guard_ok(ob, o.numel()) and _guard_ok(lb, lse.numel()), "write outside the outputs"
    ro, rl = oracle.attn_fwd_varlen(wl.bits(q), wl.bits(k), wl.bits(v), cq.numpy(), ck.numpy(),
                                    wl.DTYPE_CODE[dtype], scale, causal)
    check(o, lse, ro, rl, dtype, "varlen %s" % ((q_lens, k_lens, Hq, Hkv, d, dtype, causal),))


def test_fwd_varlen_full_size_sampled():
    """The bench's packed batch (8192 tokens, lengths U[256, 4096], Hq = Hkv = 32,
    d = 128, causal), sampled rows of every sequence against the oracle."""
    lens = wl.varlen_lengths(8192, 256, 4096, seed=1)
    q, k, v, cq, ck = wl.varlen_inputs(lens, lens, 32, 32, 128, "bf16", seed=1)
    scale = 1.0 / math.sqrt(128)
    o, lse = ea.fwd_varlen(*_dev(q, k, v, cq, ck), max(lens), causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    o, lse = o.cpu(), lse.cpu()
    for b, n in enumerate(lens):
        s0 = int(cq[b])
        qb = q[s0:s0 + n].transpose(0, 1)[None].contiguous()
        kb = k[s0:s0 + n].transpose(0, 1)[None].contiguous()
        vb = v[s0:s0 + n].transpose(0, 1)[None].contiguous()
        rows = _sample_rows(1, 32, n, 3, 77 + b)
        ro, rl = oracle.attn_fwd_rows(wl.bits(qb), wl.bits(kb), wl.bits(vb), 0, scale, True, rows)
        og = o[s0 + rows[:, 2], rows[:, 1]]
        lg = lse[rows[:, 1], s0 + rows[:, 2]]
        check(og, lg, ro, rl, "bf16", "varlen full size, sequence %d (N=%d)" % (b, n))


# --------------------------------------------------------------- backward

# Gradient tolerance (none is set for gradients elsewhere), derived from the
# kernels' arithmetic in tests/grad_bound.py: every element has its own bound,
# built from where the gradient kernels round (P and dS to the input dtype before
# their products, D from the forward's rounded output, fp32 sums, the rounded
# outputs), with independent roundings summed in the probabilistic (8 sigma)
# form. As a second, coarser check the largest error of a tensor stays below
# bf16 2^-6 / fp16 2^-8 of its largest reference gradient.
TOL_GRAD = {"bf16": 2.0 ** -6, "fp16": 2.0 ** -8}

BWD = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, causal
    (1, 2, 2, 128, 128, 64, "fp16", True),
    (1, 2, 2, 128, 128, 64, "fp16", False),
    (2, 4, 2, 200, 200, 128, "bf16", True),
    (1, 8, 2, 300, 100, 128, "bf16", True),
    (1, 4, 4, 100, 300, 128, "bf16", True),
    (1, 4, 1, 257, 257, 64, "bf16", False),
    (1, 4, 4, 1000, 1000, 128, "bf16", True),
    (1, 4, 4, 2048, 2048, 128, "bf16", True),
    # 8 and 16 (batch, head) units: the XCD-contiguous block order of both
    # gradient kernels, with GQA and a ragged length
    (2, 8, 4, 333, 333, 128, "bf16", True),
    # GQA 4:1 with more keys than rows (bottom-right causal alignment) and the
    # reverse, over several 256-row dQ workgroups and 128-key dK/dV workgroups
    (1, 16, 4, 700, 1500, 128, "fp16", True),
    (2, 8, 2, 1100, 600, 64, "bf16", True),
    (1, 8, 8, 1536, 1536, 64, "fp16", False),
]


def _check_grad(g_gpu, g_ref, bound, dtype, what):
    g = g_gpu.detach().float().cpu().double().numpy()
    assert np.isfinite(g).all(), "%s: NaN/Inf" % what
    err = np.abs(g - g_ref)
    scale = max(1e-30, np.abs(g_ref).max())
    ratio = np.where(bound > 0, err / np.maximum(bound, 1e-300), np.where(err > 0, np.inf, 0.0))
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    print("%s: max err %.3e (%.3e of max |ref| %.3e), max err/bound %.3f at %s" %
          (what, err.max(), err.max() / scale, scale, ratio.max(), worst))
    assert ratio.max() <= 1.0, "%s: error %.3e above its bound %.3e at %s (ref %.4e, gpu %.4e)" % (
        what, err[worst], bound[worst], worst, g_ref[worst], g[worst])
    assert err.max() <= TOL_GRAD[dtype] * scale, "%s: %s" % (what, _report(err, g_ref))


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal", BWD)
def test_backward(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    seed = zlib.crc32(repr(("bwd", B, Hq, Hkv, Nq, Nk, d, dtype, causal)).encode()) % 10000
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod = _dev(q, k, v, do)
    o, lse = ea.fwd(qd, kd, vd, causal=causal, scale=scale)
    outs = [_guarded(t.shape, t.dtype) for t in (qd, kd, vd)]
    deltab, delta = _guarded(tuple(lse.shape), torch.float32)
    ea.attn_bwd(qd, kd, vd, o, dod, lse, delta, outs[0][1], outs[1][1], outs[2][1], causal,
                scale)
    torch.cuda.synchronize()
    for buf, t in outs + [(deltab, delta)]:
        assert _guard_ok(buf, t.numel()), "write outside an output"
    rq, rk, rv = oracle.attn_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do),
                                 wl.DTYPE_CODE[dtype], scale, causal)
    bq, bk, bv = grad_bound(q, k, v, do, dtype, scale, causal)
    tag = "bwd %s" % ((B, Hq, Hkv, Nq, Nk, d, dtype, causal),)
    _check_grad(outs[0][1], rq, bq, dtype, tag + " dq")
    _check_grad(outs[1][1], rk, bk, dtype, tag + " dk")
    _check_grad(outs[2][1], rv, bv, dtype, tag + " dv")


def _run_bwd_both(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    """attn_bwd and attn_bwd_ds on one case, each against the oracle with the
    per-element gradient bound."""
    seed = zlib.crc32(repr(("bwd-steps", B, Hq, Hkv, Nq, Nk, d, dtype, causal)).encode()) % 10000
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod = _dev(q, k, v, do)
    o, lse = ea.fwd(qd, kd, vd, causal=causal, scale=scale)
    rq, rk, rv = oracle.attn_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do),
                                 wl.DTYPE_CODE[dtype], scale, causal)
    bq, bk, bv = grad_bound(q, k, v, do, dtype, scale, causal)
    for form in ("bwd", "bwd_ds"):
        outs = [_guarded(t.shape, t.dtype) for t in (qd, kd, vd)]
        deltab, delta = _guarded(tuple(lse.shape), torch.float32)
        if form == "bwd":
            ea.attn_bwd(qd, kd, vd, o, dod, lse, delta, outs[0][1], outs[1][1], outs[2][1],
                        causal, scale)
        else:
            ds = torch.full((ea.attn_bwd_ds_workspace(B, Hq, Nq, Nk),), 0xFF, dtype=torch.uint8,
                            device="cuda")
            ea.attn_bwd_ds(qd, kd, vd, o, dod, lse, delta, ds, outs[0][1], outs[1][1],
                           outs[2][1], causal, scale)
        torch.cuda.synchronize()
        for buf, t in outs + [(deltab, delta)]:
            assert _guard_ok(buf, t.numel()), "write outside an output"
        tag = "%s %s" % (form, (B, Hq, Hkv, Nq, Nk, d, dtype, causal))
        _check_grad(outs[0][1], rq, bq, dtype, tag + " dq")
        _check_grad(outs[1][1], rk, bk, dtype, tag + " dk")
        _check_grad(outs[2][1], rv, bv, dtype, tag + " dv")


# The dK/dV kernel walks 64-row steps (every query head of a GQA group) in a
# three-slot ring, with its first and last iterations compiled apart from the
# steady-state loop: non-causal cases with Nq = 64 n and one 128-key block give
# every workgroup exactly n (or group * n) steps, so these cover each step count
# from 1 to 8 and each slot the loop can end on, for both roles.
BWD_STEPS = ([(1, 2, 2, 64 * n, 128, 128, "bf16", False) for n in range(1, 8)] +
             [(1, 4, 2, 64 * n, 96, 64, "fp16", False) for n in (1, 2, 3, 4)] +
             [(1, 2, 2, 64 * 5 - 17, 128, 128, "bf16", False),
              (2, 2, 1, 64 * 3, 128, 64, "bf16", True),
              # one row and one key; a short causal block against a long key range
              # (workgroups whose keys no row sees take no step at all)
              (1, 2, 2, 1, 1, 128, "bf16", True),
              (1, 2, 1, 17, 300, 64, "fp16", True)])


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal", BWD_STEPS)
def test_backward_step_counts(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    _run_bwd_both(B, Hq, Hkv, Nq, Nk, d, dtype, causal)


# The dQ kernel's 256-row workgroups walk 32-key blocks of 64-key tiles staged
# three slots deep, its two waves per SIMD one phase apart: every tile count from
# 1 to 7 (each slot reused, the unrolled six-block loop entered and left at each
# offset), key counts that end half-way into a tile (a last block with no key),
# and causal blocks whose waves see different numbers of blocks (rows past the
# keys' range see none: the workgroup takes no block at all).
DQ_BLOCKS = ([(1, 2, 1, 256, 64 * n, 128, "bf16", False) for n in range(1, 8)] +
             [(1, 2, 2, 256, 32 * n + 1, 64, "fp16", False) for n in (1, 4, 9)] +
             [(1, 2, 2, 256 + 64 * n, 256 + 64 * n, 128, "bf16", True) for n in (0, 1, 3)] +
             [(1, 4, 1, 300, 97, 128, "bf16", True), (1, 2, 2, 520, 250, 64, "bf16", True)])


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal", DQ_BLOCKS)
def test_backward_dq_block_counts(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    _run_bwd_both(B, Hq, Hkv, Nq, Nk, d, dtype, causal)


# Head counts at which the gradient kernels deal their workgroups to the XCDs in
# groups of units (a multiple of 8 units per XCD and of the group size), checked
# whole against the oracle: every (unit, block) pair must be computed exactly once.
BWD_GROUPED = [(1, 64, 64, 512, 512, 64, "bf16", True),
               (1, 64, 16, 300, 300, 128, "fp16", True),
               (2, 32, 32, 256, 256, 64, "bf16", False)]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal", BWD_GROUPED)
def test_backward_grouped_order(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    _run_bwd_both(B, Hq, Hkv, Nq, Nk, d, dtype, causal)


def test_backward_full_size_sampled_heads():
    """The backward on the whole llm_prefill workload, in the launch configuration
    the benchmark times; three (batch, head) slices, first and last included, are
    checked against the oracle's backward of that head alone (heads are independent
    when Hq == Hkv)."""
    w = wl.WORKLOADS["llm_prefill"]
    assert w.Hq == w.Hkv
    q, k, v = wl.workload_prefill_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 7)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    qd, kd, vd, dod = _dev(q, k, v, do)
    o, lse = ea.fwd(qd, kd, vd, causal=True, scale=w.scale)
    dq, dk, dv = ea.bwd(qd, kd, vd, o, lse, dod, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    picks = [(0, 0), (w.B - 1, w.Hq - 1), (int(rng.integers(w.B)), int(rng.integers(w.Hq)))]
    for b, h in picks:
        sl = lambda t: t[b:b + 1, h:h + 1].contiguous()
        rq, rk, rv = oracle.attn_bwd(wl.bits(sl(q)), wl.bits(sl(k)), wl.bits(sl(v)),
                                     wl.bits(sl(do)), wl.DTYPE_CODE[w.dtype], w.scale, True)
        bq, bk, bv = grad_bound(sl(q), sl(k), sl(v), sl(do), w.dtype, w.scale, True)
        tag = "bwd llm_prefill b=%d h=%d" % (b, h)
        _check_grad(sl(dq.cpu()), rq, bq, w.dtype, tag + " dq")
        _check_grad(sl(dk.cpu()), rk, bk, w.dtype, tag + " dk")
        _check_grad(sl(dv.cpu()), rv, bv, w.dtype, tag + " dv")


# --------------------------------------------------------------- backward through a stored dS

BWD_DS = BWD + [
    # Nq != Nk with causal alignment: the dK/dV workgroups leave dS^T entries of
    # rows above their first step unwritten; the dQ kernel must mask them
    (1, 4, 2, 200, 500, 128, "bf16", True),
    (1, 4, 4, 500, 200, 64, "fp16", True),
    (2, 4, 4, 130, 70, 128, "bf16", True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal", BWD_DS)
def test_backward_ds(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    """attn_bwd_ds against the oracle (the same per-element bound as attn_bwd), with
    the dS workspace filled with NaN bit patterns first, so that a read of an entry
    the dK/dV kernel did not write would show."""
    seed = zlib.crc32(repr(("bwd", B, Hq, Hkv, Nq, Nk, d, dtype, causal)).encode()) % 10000
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod = _dev(q, k, v, do)
    o, lse = ea.fwd(qd, kd, vd, causal=causal, scale=scale)
    outs = [_guarded(t.shape, t.dtype) for t in (qd, kd, vd)]
    deltab, delta = _guarded(tuple(lse.shape), torch.float32)
    n = ea.attn_bwd_ds_workspace(B, Hq, Nq, Nk)
    assert n == B * Hq * ((Nk + 63) // 64) * ((Nq + 127) // 128) * 16384
    ds = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    ea.attn_bwd_ds(qd, kd, vd, o, dod, lse, delta, ds, outs[0][1], outs[1][1], outs[2][1],
                   causal, scale)
    torch.cuda.synchronize()
    for buf, t in outs + [(deltab, delta)]:
        assert _guard_ok(buf, t.numel()), "write outside an output"
    rq, rk, rv = oracle.attn_bwd(wl.bits(q), wl.bits(k), wl.bits(v), wl.bits(do),
                                 wl.DTYPE_CODE[dtype], scale, causal)
    bq, bk, bv = grad_bound(q, k, v, do, dtype, scale, causal)
    tag = "bwd_ds %s" % ((B, Hq, Hkv, Nq, Nk, d, dtype, causal),)
    _check_grad(outs[0][1], rq, bq, dtype, tag + " dq")
    _check_grad(outs[1][1], rk, bk, dtype, tag + " dk")
    _check_grad(outs[2][1], rv, bv, dtype, tag + " dv")
    if causal and Nq > Nk:
        assert not outs[0][1][:, :, : Nq - Nk].any(), "rows with no key must get dq = 0"


def test_backward_ds_full_size_sampled_heads():
    """attn_bwd_ds on the whole llm_prefill workload (as the benchmark runs it), three
    (batch, head) slices against the oracle's backward of that head alone."""
    w = wl.WORKLOADS["llm_prefill"]
    q, k, v = wl.workload_prefill_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 7)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    qd, kd, vd, dod = _dev(q, k, v, do)
    o, lse = ea.fwd(qd, kd, vd, causal=True, scale=w.scale)
    dq, dk, dv = ea.bwd_ds(qd, kd, vd, o, lse, dod, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 1)
    picks = [(0, 0), (w.B - 1, w.Hq - 1), (int(rng.integers(w.B)), int(rng.integers(w.Hq)))]
    for b, h in picks:
        sl = lambda t: t[b:b + 1, h:h + 1].contiguous()
        rq, rk, rv = oracle.attn_bwd(wl.bits(sl(q)), wl.bits(sl(k)), wl.bits(sl(v)),
                                     wl.bits(sl(do)), wl.DTYPE_CODE[w.dtype], w.scale, True)
        bq, bk, bv = grad_bound(sl(q), sl(k), sl(v), sl(do), w.dtype, w.scale, True)
        tag = "bwd_ds llm_prefill b=%d h=%d" % (b, h)
        _check_grad(sl(dq.cpu()), rq, bq, w.dtype, tag + " dq")
        _check_grad(sl(dk.cpu()), rk, bk, w.dtype, tag + " dk")
        _check_grad(sl(dv.cpu()), rv, bv, w.dtype, tag + " dv")


# --------------------------------------------------------------- one-call decode (library chunk)

AUTO = [
    # B, Hq, Hkv, d, dtype, lens (None: drawn on [1, max_len]), max_len
    (256, 32, 8, 128, "bf16", None, 512),        # one pass: 2048 items fill the waves
    (64, 32, 8, 128, "bf16", None, 512),         # split into 256-key chunks + combine
    (300, 8, 8, 64, "fp16", [0, 1, 300] * 100, 300),  # one pass, empty sequences included
    (16, 32, 8, 128, "bf16", None, 2048),
    # one pass, 8 192 items of one 32-key tile each: every wave walks eight of them
    (1024, 32, 8, 128, "bf16", None, 32),
    # one pass, items of one or two tiles, four per wave
    (512, 8, 8, 128, "bf16", None, 64),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,dtype,lens,max_len", AUTO)
def test_decode_one_call(B, Hq, Hkv, d, dtype, lens, max_len):
    seed = 3000 + B + max_len + d
    sl, q, kc, vc = wl.decode_inputs(B, Hq, Hkv, d, dtype, seed, l_min=1, l_max=max_len,
                                     max_len=max_len, device="cpu", seq_lens=lens)
    scale = 1.0 / math.sqrt(d)
    qd, kcd, vcd, sld = _dev(q, kc, vc, sl)
    n = ea.attn_decode_workspace(B, Hq, Hkv, max_len, d)
    wsb, ws = _guarded((max(n, 1),), torch.float32)
    ob, o = _guarded((B, Hq, d), q.dtype)
    lb, lse = _guarded((B, Hq), torch.float32)
    ea.attn_decode(qd, kcd, vcd, sld, o, lse, ws if n else None, scale)
    torch.cuda.synchronize()
    for buf, t in ((wsb, ws), (ob, o), (lb, lse)):
        assert _guard_ok(buf, t.numel()), "write outside an output or the workspace"
    ro, rl = oracle.decode(wl.bits(q), wl.bits(kc), wl.bits(vc), sl.numpy(), wl.DTYPE_CODE[dtype],
                           scale)
    # Sequences of at most 64 keys give outputs close to single V rows (|O| up
    # to about 4.5), where bf16 rounding alone exceeds the gate: judge the excess.
    check(o, lse, ro, rl, dtype, "one-call decode (workspace %d floats)" % n,
          floor_aware=max_len <= 64)


def test_decode_one_call_workspace_sizes():
    # decode workload: 2048-key chunks -> 16 chunk slots; short batch: one pass
    assert ea.attn_decode_workspace(64, 32, 8, 32768, 128) == 64 * 32 * 16 * 129
    assert ea.attn_decode_workspace(256, 32, 8, 512, 128) == 0
    with pytest.raises(ea.AttnError):
        ea.attn_decode_workspace(2, 6, 4, 64, 128)


def test_decode_one_call_full_size_sampled():
    w = wl.WORKLOADS["decode"]
    sl, q, kc, vc = wl.workload_decode_inputs(w, device="cuda")
    qd, sld = q.cuda(), sl.cuda()
    o, lse = ea.decode_auto(qd, kc, vc, sld, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    lens = sl.numpy()
    for b in sorted({int(np.argmax(lens)), int(np.argmin(lens)), 7, 50}):
        L = int(lens[b])
        ro, rl = oracle.decode(wl.bits(q[b:b + 1]), wl.bits(kc[b:b + 1, :, :L].cpu()),
                               wl.bits(vc[b:b + 1, :, :L].cpu()), np.array([L], dtype=np.int32),
                               0, w.scale)
        check(o[b:b + 1], lse[b:b + 1], ro, rl, "bf16", "one-call decode seq %d (L=%d)" % (b, L))


# --------------------------------------------------------------- local (sliding-window) attention

LOCAL = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, window_left, window_right
    (1, 4, 2, 500, 500, 128, "bf16", 63, 0),
    (1, 4, 2, 500, 500, 128, "bf16", 64, 0),
    (1, 4, 4, 700, 700, 64, "fp16", 100, 0),
    (2, 4, 2, 1000, 1000, 128, "bf16", 256, 0),
    (1, 4, 4, 300, 300, 128, "bf16", 0, 0),
    (1, 8, 2, 600, 600, 128, "bf16", 128, 128),
    (1, 4, 4, 257, 513, 128, "bf16", 200, 0),
    (1, 4, 4, 513, 257, 128, "bf16", 50, 10),
    (1, 4, 4, 400, 400, 64, "bf16", -1, 0),
    (1, 4, 4, 400, 400, 128, "bf16", 300, -1),
    (1, 2, 2, 2048, 2048, 128, "bf16", 512, 0),
    # windows above 1024 keys (or open on one side) take the one-group form,
    # the others the two-halves form: both, at d = 64 and 128
    (1, 4, 4, 2048, 2048, 128, "bf16", 1500, 0),
    (1, 4, 2, 700, 700, 64, "fp16", 1000, 24),
    (2, 4, 4, 1000, 1000, 64, "bf16", 1000, 25),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,left,right", LOCAL)
def test_fwd_local(B, Hq, Hkv, Nq, Nk, d, dtype, left, right):
    seed = zlib.crc32(repr(("local", B, Hq, Hkv, Nq, Nk, d, dtype, left, right)).encode()) % 10000
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed)
    scale = 1.0 / math.sqrt(d)
    ob, o = _guarded(q.shape, q.dtype)
    lb, lse = _guarded((B, Hq, Nq), torch.float32)
    ea.attn_fwd_local(*_dev(q, k, v), o, lse, left, right, scale)
    torch.cuda.synchronize()
    assert _guard_ok(ob, o.numel()) and _guard_ok(lb, lse.numel()), "write outside the outputs"
    ro, rl = oracle.attn_fwd_local(wl.bits(q), wl.bits(k), wl.bits(v), wl.DTYPE_CODE[dtype], scale,
                                   left, right)
    check(o, lse, ro, rl, dtype, "local %s" % ((B, Hq, Hkv, Nq, Nk, d, dtype, left, right),))


# --------------------------------------------------------------- packed qkv input

QKV = [
    # B, N, H, d, dtype, causal
    (2, 300, 4, 128, "bf16", True),
    (1, 129, 2, 64, "fp16", False),
    (1, 1000, 8, 128, "bf16", True),
]


@pytest.mark.parametrize("B,N,H,d,dtype,causal", QKV)
def test_fwd_qkvpacked(B, N, H, d, dtype, causal):
    seed = zlib.crc32(repr(("qkv", B, N, H, d, dtype, causal)).encode()) % 10000
    g = torch.Generator().manual_seed(seed)
    qkv = torch.randn((B, N, 3, H, d), generator=g).to(wl.DTYPES[dtype])
    scale = 1.0 / math.sqrt(d)
    ob, o = _guarded((B, N, H, d), qkv.dtype)
    lb, lse = _guarded((B, H, N), torch.float32)
    qkvd = qkv.cuda()
    ea.attn_fwd_qkvpacked(qkvd, o, lse, causal, scale)
    torch.cuda.synchronize()
    assert _guard_ok(ob, o.numel()) and _guard_ok(lb, lse.numel()), "write outside the outputs"
    ro, rl = oracle.attn_fwd_qkvpacked(wl.bits(qkv), wl.DTYPE_CODE[dtype], scale, causal)
    check(o, lse, ro, rl, dtype, "qkvpacked %s" % ((B, N, H, d, dtype, causal),))
    # same tiles and arithmetic as the dense kernel on the unpacked tensors
    q, k, v = (qkvd[:, :, i].transpose(1, 2).contiguous() for i in range(3))
    od, ld = ea.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(od.transpose(1, 2).contiguous().view(torch.int16), o.view(torch.int16))
    assert torch.equal(ld, lse)


# --------------------------------------------------------------- maximum lengths

MAX_SEQ = 1 << 23  # the longest sequence the C ABI accepts


def test_fwd_maximum_key_length():
    """Nk at the ABI's limit: one head's K and V are 2 GiB each, so its per-head byte
    offsets reach 2^31. 192 causal rows aligned to the bottom-right corner (the last
    row sees every key), four rows checked against the oracle."""
    Nq, Nk, d = 192, MAX_SEQ, 128
    g = torch.Generator(device="cuda").manual_seed(1234)
    q = torch.randn((1, 1, Nq, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, 1, Nk, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, 1, Nk, d), generator=g, device="cuda").to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fwd(q, k, v, True, scale)
    rows = np.array([[0, 0, 0], [0, 0, 1], [0, 0, 100], [0, 0, Nq - 1]], dtype=np.int64)
    ro, rl = oracle.attn_fwd_rows(wl.bits(q.cpu()), wl.bits(k.cpu()), wl.bits(v.cpu()), 0,
                                  scale, True, rows)
    check(o[0, 0, rows[:, 2]], lse[0, 0, rows[:, 2]], ro, rl, "bf16",
          "forward, Nk = 2^23 (rows 0, 1, 100, 191)")


def test_decode_maximum_length():
    """One sequence of 2^23 keys (the ABI's limit: 2 GiB of K and of V for its
    kv-head) through the split + combine (16384 chunks of 512 keys), the one-call and
    the fused decode, each against the oracle."""
    Hq, Hkv, d = 4, 1, 128
    g = torch.Generator(device="cuda").manual_seed(4321)
    q = torch.randn((1, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.randn((1, Hkv, MAX_SEQ, d), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((1, Hkv, MAX_SEQ, d), generator=g, device="cuda").to(torch.bfloat16)
    sl = torch.tensor([MAX_SEQ], dtype=torch.int32)
    sld = sl.cuda()
    scale = 1.0 / math.sqrt(d)
    ro, rl = oracle.decode(wl.bits(q.cpu()), wl.bits(kc.cpu()), wl.bits(vc.cpu()), sl.numpy(),
                           0, scale)
    o, lse = ea.decode(q, kc, vc, sld, chunk=512, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, ro, rl, "bf16", "split + combine decode, L = 2^23")
    o, lse = ea.decode_auto(q, kc, vc, sld, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, ro, rl, "bf16", "one-call decode, L = 2^23")
    o, lse = ea.decode_fused(q, kc, vc, sld, chunk=512, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, ro, rl, "bf16", "fused decode, L = 2^23")
