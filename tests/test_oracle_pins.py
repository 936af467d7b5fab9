"""Pins of the fp64 CPU oracle to things other than itself.

Each test checks the oracle against a fact fixed by the mathematics or by an
independent routine: a library implementation (torch's fp64 scaled-dot-product
attention and logsumexp), a deliberately naive brute-force formulation written
here in numpy (no max subtraction, explicit mask matrix, full probability
matrix), closed forms (Q = 0, V constant, causal row 0, a hand-worked example in
tests/golden), and invariants (row sums, shift and permutation invariance, GQA
equals repeated-KV, decode equals one-row prefill, chunked merge equals direct).
Together they catch a dropped term, a wrong sign, an off-by-one in the mask, a
wrong head mapping or a transposed operand anywhere in the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_46_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(t):
    return wl.bits(t)


def _f64(t):
    return t.double().numpy()


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(wl.DTYPES[dtype])


def brute_force(q, k, v, scale, causal):
    """Naive fp64 attention: full score matrix, explicit mask matrix, no max
    subtraction, full probability matrix. q [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d]."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, Hq, Nq, d))
    lse = np.zeros((B, Hq, Nq))
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    allowed = (j <= i + (Nk - Nq)) if causal else np.ones((Nq, Nk), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            s = scale * (q[b, h] @ k[b, g].T)
            e = np.where(allowed, np.exp(s), 0.0)
            z = e.sum(axis=1, keepdims=True)
            with np.errstate(invalid="ignore", divide="ignore"):
                p = np.where(z > 0, e / z, 0.0)
                lse[b, h] = np.where(z[:, 0] > 0, np.log(z[:, 0]), -np.inf)
            o[b, h] = p @ v[b, g]
    return o, lse


# ---------------------------------------------------------------- decoders

def test_bf16_decoder_matches_torch_for_every_pattern():
    pats = np.arange(65536, dtype=np.uint16)
    got = oracle.decode_values(pats, oracle.BF16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_fp16_decoder_matches_numpy_for_every_pattern():
    pats = np.arange(65536, dtype=np.uint16)
    got = oracle.decode_values(pats, oracle.FP16)
    ref = pats.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- golden example

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_hand_worked_example(dtype, causal):
    with open(os.path.join(GOLDEN, "closed_form_two_keys.json")) as f:
        g = json.load(f)
    t = wl.DTYPES[dtype]
    q = torch.tensor(g["q"], dtype=torch.float32).to(t).view(1, 1, 2, 2)
    k = torch.tensor(g["k"], dtype=torch.float32).to(t).view(1, 1, 2, 2)
    v = torch.tensor(g["v"], dtype=torch.float32).to(t).view(1, 1, 2, 2)
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), wl.DTYPE_CODE[dtype], g["scale"],
                             causal)
    exp = g["expected"]["causal" if causal else "noncausal"]
    env = {"exp": math.exp, "log": math.log}
    want_o = np.array([[eval(x, env) for x in row] for row in exp["o"]])
    want_lse = np.array([eval(x, env) for x in exp["lse"]])
    np.testing.assert_allclose(o[0, 0], want_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], want_lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [("fp16", 64), ("bf16", 128), ("bf16", 16)])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1), (8, 2)])
def test_matches_torch_sdpa_fp64(causal, dtype, d, Hq, Hkv):
    B, N = 2, 37
    q = _rand((B, Hq, N, d), dtype, 1)
    k = _rand((B, Hkv, N, d), dtype, 2)
    v = _rand((B, Hkv, N, d), dtype, 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), wl.DTYPE_CODE[dtype], scale, causal)
    rep = Hq // Hkv
    kd = k.double().repeat_interleave(rep, dim=1)
    vd = v.double().repeat_interleave(rep, dim=1)
    sc = float(np.float32(scale))
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), kd, vd,
                                                           is_causal=causal, scale=sc)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = sc * (q.double() @ kd.transpose(-1, -2))
    if causal:
        mask = torch.ones(N, N, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (5, 5), (7, 19), (19, 7), (32, 32), (3, 30)])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (6, 3)])
def test_matches_brute_force(causal, Nq, Nk, Hq, Hkv):
    d = 8
    q = _rand((2, Hq, Nq, d), "bf16", 10)
    k = _rand((2, Hkv, Nk, d), "bf16", 11)
    v = _rand((2, Hkv, Nk, d), "bf16", 12)
    scale = 0.35
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, scale, causal)
    ro, rl = brute_force(_f64(q), _f64(k), _f64(v), float(np.float32(scale)), causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    fin = np.isfinite(rl)
    np.testing.assert_allclose(lse[fin], rl[fin], rtol=0, atol=1e-12)


def test_fully_masked_rows_are_zero_with_minus_inf_lse():
    # Bottom-right causal with Nq > Nk: rows i < Nq - Nk have no allowed key.
    Nq, Nk, d = 10, 4, 8
    q = _rand((1, 1, Nq, d), "bf16", 20)
    k = _rand((1, 1, Nk, d), "bf16", 21)
    v = _rand((1, 1, Nk, d), "bf16", 22)
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.5, True)
    assert np.all(o[0, 0, :Nq - Nk] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, :Nq - Nk]))
    assert np.all(np.isfinite(lse[0, 0, Nq - Nk:]))
    # the first row that sees anything sees exactly key 0
    np.testing.assert_array_equal(o[0, 0, Nq - Nk], _f64(v)[0, 0, 0])


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_prefix_mean_and_log_count(causal):
    N, d = 33, 16
    q = torch.zeros((1, 2, N, d), dtype=torch.bfloat16)
    k = _rand((1, 2, N, d), "bf16", 30)
    v = _rand((1, 2, N, d), "bf16", 31)
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.125, causal)
    vd = _f64(v)
    for i in range(N):
        n = i + 1 if causal else N
        np.testing.assert_allclose(o[0, :, i], vd[0, :, :n].mean(axis=1), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=0, atol=1e-13)


def test_zero_keys_gives_the_same_as_zero_query():
    N, d = 20, 16
    q = _rand((1, 1, N, d), "bf16", 32)
    k = torch.zeros((1, 1, N, d), dtype=torch.bfloat16)
    v = _rand((1, 1, N, d), "bf16", 33)
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.125, True)
    vd = _f64(v)
    for i in range(N):
        np.testing.assert_allclose(o[0, 0, i], vd[0, 0, :i + 1].mean(axis=0), atol=1e-13)
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_constant_value_rows_give_that_constant(causal):
    N, d = 40, 16
    q = _rand((1, 2, N, d), "bf16", 40, 3.0)
    k = _rand((1, 2, N, d), "bf16", 41, 3.0)
    c = torch.linspace(-2, 2, d).to(torch.bfloat16)
    v = c.expand(1, 2, N, d).contiguous()
    o, _ = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.3, causal)
    np.testing.assert_allclose(o, np.broadcast_to(c.double().numpy(), o.shape), rtol=0,
                               atol=1e-12)


def test_causal_row_zero_is_first_value_row():
    N, d = 12, 16
    q = _rand((1, 1, N, d), "fp16", 50)
    k = _rand((1, 1, N, d), "fp16", 51)
    v = _rand((1, 1, N, d), "fp16", 52)
    scale = 0.25
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 1, scale, True)
    np.testing.assert_array_equal(o[0, 0, 0], _f64(v)[0, 0, 0])
    s00 = scale * float(_f64(q)[0, 0, 0] @ _f64(k)[0, 0, 0])
    assert abs(lse[0, 0, 0] - s00) < 1e-13


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_expose_probabilities_that_sum_to_one(causal):
    N = d = 16
    q = _rand((1, 1, N, d), "bf16", 60, 2.0)
    k = _rand((1, 1, N, d), "bf16", 61, 2.0)
    v = torch.eye(N, d).to(torch.bfloat16).view(1, 1, N, d)
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.4, causal)
    p = o[0, 0]
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(np.triu(p, 1) == 0)
    # the log of each probability is its score minus the LSE
    s = float(np.float32(0.4)) * (_f64(q)[0, 0] @ _f64(k)[0, 0].T)
    i, j = np.nonzero(p)
    np.testing.assert_allclose(np.log(p[i, j]), s[i, j] - lse[0, 0][i], rtol=0, atol=1e-12)


def test_key_shift_leaves_output_and_shifts_lse():
    # Integer-valued fp16 inputs keep the shifted keys exact.
    N, d = 24, 8
    g = torch.Generator().manual_seed(70)
    q = torch.randint(-3, 4, (1, 1, N, d), generator=g).to(torch.float16)
    k = torch.randint(-3, 4, (1, 1, N, d), generator=g).to(torch.float16)
    v = _rand((1, 1, N, d), "fp16", 71)
    u = torch.randint(-2, 3, (d,), generator=g).to(torch.float16)
    scale = 0.25
    o1, l1 = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 1, scale, True)
    o2, l2 = oracle.attn_fwd(_bits(q), _bits(k + u), _bits(v), 1, scale, True)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    shift = scale * (_f64(q)[0, 0] @ u.double().numpy())
    np.testing.assert_allclose(l2[0, 0], l1[0, 0] + shift, rtol=0, atol=1e-12)


def test_key_value_permutation_invariance_non_causal():
    N, d = 30, 16
    q = _rand((1, 2, N, d), "bf16", 80)
    k = _rand((1, 2, N, d), "bf16", 81)
    v = _rand((1, 2, N, d), "bf16", 82)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(83))
    o1, l1 = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.25, False)
    o2, l2 = oracle.attn_fwd(_bits(q), _bits(k[:, :, perm]), _bits(v[:, :, perm]), 0, 0.25,
                             False)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


def test_gqa_equals_repeated_kv():
    B, Hq, Hkv, N, d = 2, 8, 2, 21, 16
    q = _rand((B, Hq, N, d), "bf16", 90)
    k = _rand((B, Hkv, N, d), "bf16", 91)
    v = _rand((B, Hkv, N, d), "bf16", 92)
    o1, l1 = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.25, True)
    kr = k.repeat_interleave(Hq // Hkv, dim=1)
    vr = v.repeat_interleave(Hq // Hkv, dim=1)
    o2, l2 = oracle.attn_fwd(_bits(q), _bits(kr), _bits(vr), 0, 0.25, True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_row_subset_matches_full():
    B, Hq, Hkv, N, d = 2, 4, 2, 50, 16
    q = _rand((B, Hq, N, d), "bf16", 100)
    k = _rand((B, Hkv, N, d), "bf16", 101)
    v = _rand((B, Hkv, N, d), "bf16", 102)
    o, lse = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.2, True)
    rows = np.array([[0, 0, 0], [1, 3, 49], [0, 2, 17], [1, 1, 33]], dtype=np.int64)
    ro, rl = oracle.attn_fwd_rows(_bits(q), _bits(k), _bits(v), 0, 0.2, True, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(ro[n], o[b, h, i])
        assert rl[n] == lse[b, h, i]


# ---------------------------------------------------------------- decode

def _small_decode(seed=3, B=5, Hq=8, Hkv=2, d=16, lens=(1, 9, 0, 31, 16), max_len=32,
                  dtype="bf16"):
    sl, q, kc, vc = wl.decode_inputs(B, Hq, Hkv, d, dtype, seed, l_min=0, l_max=max_len,
                                     max_len=max_len, device="cpu", seq_lens=list(lens))
    return sl.numpy(), q, kc, vc


def test_decode_equals_one_row_prefill():
    sl, q, kc, vc = _small_decode()
    o, lse = oracle.decode(_bits(q), _bits(kc), _bits(vc), sl, 0, 0.25)
    for b, L in enumerate(sl):
        if L == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        po, pl = oracle.attn_fwd(_bits(q[b:b + 1, :, None]), _bits(kc[b:b + 1, :, :L]),
                                 _bits(vc[b:b + 1, :, :L]), 0, 0.25, True)
        np.testing.assert_array_equal(o[b], po[0, :, 0])
        np.testing.assert_array_equal(lse[b], pl[0, :, 0])


def test_decode_never_reads_past_the_sequence():
    # The cache padding holds NaN; a read past L_b would poison the output.
    sl, q, kc, vc = _small_decode()
    o, lse = oracle.decode(_bits(q), _bits(kc), _bits(vc), sl, 0, 0.25)
    assert not np.isnan(o).any() and not np.isnan(lse).any()


@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 512])
def test_chunked_merge_equals_direct(chunk):
    sl, q, kc, vc = _small_decode()
    o, lse = oracle.decode(_bits(q), _bits(kc), _bits(vc), sl, 0, 0.25)
    po, pl = oracle.decode_chunks(_bits(q), _bits(kc), _bits(vc), sl, 0, chunk, 0.25)
    C = po.shape[2]
    assert C == -(-32 // chunk)
    # chunk slots past the end of each sequence are empty
    for b, L in enumerate(sl):
        nc = -(-int(L) // chunk)
        assert np.all(np.isneginf(pl[b, :, nc:])) and np.all(po[b, :, nc:] == 0)
        assert np.all(np.isfinite(pl[b, :, :nc]))
    mo, ml = oracle.combine(po, pl, sl, chunk)
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(ml), np.isneginf(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(ml[fin], lse[fin], rtol=0, atol=1e-12)


def test_combine_of_a_single_chunk_is_identity_and_ignores_minus_inf():
    rng = np.random.default_rng(0)
    po = rng.standard_normal((1, 2, 3, 4))
    pl = np.array([[[0.5, -np.inf, -np.inf], [-np.inf, 1.5, -np.inf]]])
    o, lse = oracle.combine(po, pl, np.array([9], dtype=np.int32), 4)  # 3 chunk slots
    np.testing.assert_allclose(o[0, 0], po[0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(o[0, 1], po[0, 1, 1], atol=1e-15)
    np.testing.assert_allclose(lse[0], [0.5, 1.5], atol=1e-15)


def test_combine_two_chunks_closed_form():
    # Two chunks with LSE ln 1 and ln 3: weights 1/4 and 3/4, total LSE ln 4.
    po = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    pl = np.array([[[0.0, math.log(3.0)]]])
    o, lse = oracle.combine(po, pl, np.array([2], dtype=np.int32), 1)
    np.testing.assert_allclose(o[0, 0], [0.25, 0.75], atol=1e-15)
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-15


@pytest.mark.parametrize("page_size", [16, 32, 48, 512])
def test_paged_decode_equals_decode_of_the_logical_cache(page_size):
    """A paged cache holds the same keys as the padded cache it was scattered
    from (numpy/torch scatter in the input module, not the oracle), so the paged
    decode must reproduce the padded decode exactly, and torch's fp64 SDPA on
    the logical keys."""
    lens = [0, 1, page_size - 1, page_size, page_size + 1, 3 * page_size + 5, 100]
    sl, q, kc, vc = wl.decode_inputs(len(lens), 8, 2, 64, "bf16", 21, max_len=max(lens) + 7,
                                     seq_lens=lens)
    kp, vp, table = wl.paged_from_padded(kc, vc, sl, page_size, seed=5)
    ro, rl = oracle.decode(_bits(q), _bits(kc), _bits(vc), sl.numpy(), 0, 0.125)
    po, pl = oracle.decode_paged(_bits(q), _bits(kp), _bits(vp), table.numpy(), sl.numpy(), 0,
                                 0.125)
    assert np.array_equal(ro, po) and np.array_equal(rl, pl)
    b = 5  # longest sequence: library routine on its logical keys
    L = lens[b]
    qt = q[b].double()[:, None, None, :]            # [Hq,1,1,d]
    kt = kc[b, :, :L].double().repeat_interleave(4, dim=0)[:, None]  # [Hq,1,L,d]
    vt = vc[b, :, :L].double().repeat_interleave(4, dim=0)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.125)
    assert np.abs(po[b] - ref[:, 0, 0].numpy()).max() < 1e-12


def test_paged_decode_with_shared_prefix_pages():
    """Two sequences whose tables list the same first pages (a shared prompt)
    see the same keys there: the result equals the padded decode of a cache in
    which the shared rows are copied into both sequences."""
    ps, d, Hkv = 32, 64, 2
    g = torch.Generator().manual_seed(9)
    pool_k = torch.randn((6, ps, Hkv, d), generator=g).to(torch.bfloat16)
    pool_v = torch.randn((6, ps, Hkv, d), generator=g).to(torch.bfloat16)
    q = torch.randn((2, 4, d), generator=g).to(torch.bfloat16)
    table = torch.tensor([[4, 1, 3], [4, 1, 0]], dtype=torch.int32)
    lens = torch.tensor([80, 70], dtype=torch.int32)
    kc = torch.full((2, Hkv, 96, d), float("nan"), dtype=torch.bfloat16)
    vc = kc.clone()
    for b in range(2):
        for j in range(int(lens[b])):
            pg = int(table[b, j // ps])
            kc[b, :, j] = pool_k[pg, j % ps]
            vc[b, :, j] = pool_v[pg, j % ps]
    ro, rl = oracle.decode(_bits(q), _bits(kc), _bits(vc), lens.numpy(), 0, 0.125)
    po, pl = oracle.decode_paged(_bits(q), _bits(pool_k), _bits(pool_v), table.numpy(),
                                 lens.numpy(), 0, 0.125)
    assert np.array_equal(ro, po) and np.array_equal(rl, pl)


def test_paged_decode_rejects_out_of_range_pages_and_ignores_unused_slots():
    sl, q, kc, vc = wl.decode_inputs(2, 4, 2, 64, "bf16", 3, max_len=64, seq_lens=[40, 17])
    kp, vp, table = wl.paged_from_padded(kc, vc, sl, 16, seed=1)
    t = table.numpy().copy()
    assert (t[1, 2:] == -1).all()  # unused slots hold -1 and are never looked up
    oracle.decode_paged(_bits(q), _bits(kp), _bits(vp), t, sl.numpy(), 0, 0.125)
    t[0, 1] = kp.shape[0]
    with pytest.raises(ValueError):
        oracle.decode_paged(_bits(q), _bits(kp), _bits(vp), t, sl.numpy(), 0, 0.125)


VARLEN_CASES = [
    # q_lens, k_lens, Hq, Hkv, causal
    ([5, 0, 17, 1, 33], [5, 0, 17, 1, 33], 4, 2, True),
    ([3, 20, 7], [10, 20, 30], 4, 4, True),      # Nq < Nk: bottom-right alignment
    ([9, 4], [2, 0], 2, 1, True),               # Nq > Nk, and a sequence with no keys
    ([12, 30, 1], [40, 5, 9], 6, 3, False),
]


@pytest.mark.parametrize("q_lens,k_lens,Hq,Hkv,causal", VARLEN_CASES)
def test_varlen_equals_each_sequence_alone(q_lens, k_lens, Hq, Hkv, causal):
    """A packed batch is B independent problems: every sequence's rows equal the
    dense oracle (itself pinned to SDPA and brute force) run on that sequence
    alone, and rows with no allowed key are O = 0, LSE = -inf."""
    q, k, v, cq, ck = wl.varlen_inputs(q_lens, k_lens, Hq, Hkv, 32, "bf16", 13)
    o, lse = oracle.attn_fwd_varlen(_bits(q), _bits(k), _bits(v), cq.numpy(), ck.numpy(), 0,
                                    0.2, causal)
    for b in range(len(q_lens)):
        qs, qe, ks, ke = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        if qe == qs:
            continue
        if ke == ks:
            assert (o[qs:qe] == 0).all() and np.isneginf(lse[:, qs:qe]).all()
            continue
        qb = q[qs:qe].transpose(0, 1)[None].contiguous()
        kb = k[ks:ke].transpose(0, 1)[None].contiguous()
        vb = v[ks:ke].transpose(0, 1)[None].contiguous()
        ro, rl = oracle.attn_fwd(_bits(qb), _bits(kb), _bits(vb), 0, 0.2, causal)
        assert np.array_equal(o[qs:qe], ro[0].transpose(1, 0, 2))
        assert np.array_equal(lse[:, qs:qe], rl[0])


def test_varlen_matches_brute_force_with_uneven_lengths():
    q_lens, k_lens = [7, 3], [11, 3]
    q, k, v, cq, ck = wl.varlen_inputs(q_lens, k_lens, 2, 2, 16, "fp16", 4)
    o, lse = oracle.attn_fwd_varlen(_bits(q), _bits(k), _bits(v), cq.numpy(), ck.numpy(), 1,
                                    0.25, True)
    for b in range(2):
        qs, qe, ks, ke = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        bo, bl = brute_force(_f64(q[qs:qe].transpose(0, 1)[None]),
                             _f64(k[ks:ke].transpose(0, 1)[None]),
                             _f64(v[ks:ke].transpose(0, 1)[None]), 0.25, True)
        assert np.abs(o[qs:qe] - bo[0].transpose(1, 0, 2)).max() < 1e-12
        assert np.abs(lse[:, qs:qe] - bl[0]).max() < 1e-12


def test_varlen_rejects_inconsistent_offsets():
    q, k, v, cq, ck = wl.varlen_inputs([4, 4], [4, 4], 2, 2, 16, "bf16", 1)
    bad = cq.numpy().copy()
    bad[1] = 9  # decreasing
    with pytest.raises(ValueError):
        oracle.attn_fwd_varlen(_bits(q), _bits(k), _bits(v), bad, ck.numpy(), 0, 0.25, True)


def _torch_grads(q, k, v, do, scale, causal):
    """fp64 autograd through torch's scaled_dot_product_attention (library
    routine) with an explicit bottom-right causal mask; GQA by repeating K/V,
    whose autograd sums the group's gradients."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    qt, kt, vt = (t.double().requires_grad_(True) for t in (q, k, v))
    kr = kt.repeat_interleave(Hq // Hkv, dim=1)
    vr = vt.repeat_interleave(Hq // Hkv, dim=1)
    mask = None
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = j <= i + (Nk - Nq)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kr, vr, attn_mask=mask, scale=scale)
    (o * do.double()).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


BWD_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 2, 2, 9, 9, 16, True),
    (2, 4, 2, 13, 13, 32, False),
    (1, 4, 1, 6, 15, 16, True),    # Nq < Nk, bottom-right
    (1, 2, 2, 17, 17, 64, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", BWD_CASES)
def test_backward_matches_torch_autograd_fp64(B, Hq, Hkv, Nq, Nk, d, causal):
    q = _rand((B, Hq, Nq, d), "bf16", 31)
    k = _rand((B, Hkv, Nk, d), "bf16", 32)
    v = _rand((B, Hkv, Nk, d), "bf16", 33)
    do = _rand((B, Hq, Nq, d), "bf16", 34)
    scale = float(np.float32(1.0 / math.sqrt(d)))  # the fp32 value the oracle receives
    dq, dk, dv = oracle.attn_bwd(_bits(q), _bits(k), _bits(v), _bits(do), 0, scale, causal)
    tq, tk, tv = _torch_grads(q, k, v, do, scale, causal)
    assert np.abs(dq - tq).max() < 1e-11
    assert np.abs(dk - tk).max() < 1e-11
    assert np.abs(dv - tv).max() < 1e-11


def test_backward_matches_finite_differences_of_the_forward():
    """Central differences of L = sum(dO * O), O from the forward oracle, with
    each probed input moved by one fp16 ulp either way (exact in the 16-bit
    inputs); truncation error is O(ulp^2)."""
    B, H, N, d = 1, 2, 7, 8
    q = _rand((B, H, N, d), "fp16", 41)
    k = _rand((B, H, N, d), "fp16", 42)
    v = _rand((B, H, N, d), "fp16", 43)
    do = _rand((B, H, N, d), "fp16", 44)
    scale = 0.3
    dq, dk, dv = oracle.attn_bwd(_bits(q), _bits(k), _bits(v), _bits(do), 1, scale, True)
    dof = _f64(do)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(_bits(qq), _bits(kk), _bits(vv), 1, scale, True)
        return float((o * dof).sum())

    rng = np.random.default_rng(3)
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in (B, H, N, d))
            t = {"q": q, "k": k, "v": v}[which]
            bits = t.view(torch.int16).clone()
            up, dn = t.clone(), t.clone()
            up.view(torch.int16)[idx] = bits[idx] + (1 if float(t[idx]) >= 0 else -1)
            dn.view(torch.int16)[idx] = bits[idx] - (1 if float(t[idx]) >= 0 else -1)
            h = float(up[idx]) - float(dn[idx])
            args_up = {"q": q, "k": k, "v": v}
            args_dn = dict(args_up)
            args_up[which], args_dn[which] = up, dn
            fd = (loss(**{a + a: b for a, b in args_up.items()})
                  - loss(**{a + a: b for a, b in args_dn.items()})) / h
            assert abs(fd - grad[idx]) < 1e-5 * max(1.0, abs(grad[idx])), (which, idx, fd,
                                                                            grad[idx])


def test_backward_closed_form_sums():
    """Sum over keys of dv_j equals the sum of dO over the rows that see any key
    (the rows of P sum to one); sum over keys of dk_j is zero (each row of dS
    sums to zero). Both per (b, kv-head), over the group's query heads."""
    B, Hq, Hkv, N, d = 2, 4, 2, 11, 16
    q = _rand((B, Hq, N, d), "bf16", 51)
    k = _rand((B, Hkv, N, d), "bf16", 52)
    v = _rand((B, Hkv, N, d), "bf16", 53)
    do = _rand((B, Hq, N, d), "bf16", 54)
    dq, dk, dv = oracle.attn_bwd(_bits(q), _bits(k), _bits(v), _bits(do), 0, 0.25, True)
    dof = _f64(do)
    for b in range(B):
        for g in range(Hkv):
            heads = [h for h in range(Hq) if h * Hkv // Hq == g]
            assert np.abs(dv[b, g].sum(axis=0) - dof[b, heads].sum(axis=(0, 1))).max() < 1e-12
            assert np.abs(dk[b, g].sum(axis=0)).max() < 1e-12


LOCAL_CASES = [
    # Nq, Nk, window_left, window_right
    (13, 13, 3, 0), (13, 13, 0, 0), (13, 13, 4, 2), (9, 15, 5, 0), (15, 9, 2, 1),
    (11, 11, -1, 3), (11, 11, 2, -1), (10, 10, 100, 0),
]


@pytest.mark.parametrize("Nq,Nk,wl,wr", LOCAL_CASES)
def test_local_attention_matches_banded_brute_force(Nq, Nk, wl, wr):
    """Against a numpy brute force with an explicit band mask (no max
    subtraction), and torch's fp64 SDPA with the same boolean mask."""
    B, Hq, Hkv, d = 1, 4, 2, 16
    q = _rand((B, Hq, Nq, d), "bf16", 61)
    k = _rand((B, Hkv, Nk, d), "bf16", 62)
    v = _rand((B, Hkv, Nk, d), "bf16", 63)
    o, lse = oracle.attn_fwd_local(_bits(q), _bits(k), _bits(v), 0, 0.25, wl, wr)
    i = np.arange(Nq)[:, None] + (Nk - Nq)
    j = np.arange(Nk)[None, :]
    band = np.ones((Nq, Nk), dtype=bool)
    if wl >= 0:
        band &= j >= i - wl
    if wr >= 0:
        band &= j <= i + wr
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    for h in range(Hq):
        g = h * Hkv // Hq
        s = 0.25 * qf[0, h] @ kf[0, g].T
        e = np.where(band, np.exp(s), 0.0)
        z = e.sum(axis=1)
        with np.errstate(invalid="ignore", divide="ignore"):
            ref_o = np.where(z[:, None] > 0, (e / z[:, None]) @ vf[0, g], 0.0)
            ref_l = np.where(z > 0, np.log(z), -np.inf)
        assert np.abs(o[0, h] - ref_o).max() < 1e-12
        assert np.array_equal(np.isneginf(lse[0, h]), np.isneginf(ref_l))
        fin = np.isfinite(ref_l)
        assert np.abs(lse[0, h][fin] - ref_l[fin]).max() < 1e-12
    if band.any(axis=1).all():
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.double(), k.double().repeat_interleave(2, 1), v.double().repeat_interleave(2, 1),
            attn_mask=torch.from_numpy(band), scale=0.25)
        assert np.abs(o - ref.numpy()).max() < 1e-12


def test_local_window_limits_reduce_to_causal_and_full():
    q = _rand((1, 2, 12, 16), "bf16", 71)
    k = _rand((1, 2, 12, 16), "bf16", 72)
    v = _rand((1, 2, 12, 16), "bf16", 73)
    for (wl, wr), causal in (((-1, 0), True), ((-1, -1), False), ((11, 0), True)):
        o, lse = oracle.attn_fwd_local(_bits(q), _bits(k), _bits(v), 0, 0.25, wl, wr)
        bo, bl = brute_force(_f64(q), _f64(k), _f64(v), 0.25, causal)
        assert np.abs(o - bo).max() < 1e-12 and np.abs(lse - bl).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_qkvpacked_equals_attention_of_the_unpacked_tensors(causal):
    """Unpacking is a pure permutation (done here by torch indexing): the packed
    oracle must equal the dense oracle on q, k, v taken out of qkv."""
    B, N, H, d = 2, 19, 3, 16
    qkv = _rand((B, N, 3, H, d), "bf16", 81)
    o, lse = oracle.attn_fwd_qkvpacked(_bits(qkv), 0, 0.25, causal)
    q, k, v = (qkv[:, :, i].transpose(1, 2).contiguous() for i in range(3))
    ro, rl = oracle.attn_fwd(_bits(q), _bits(k), _bits(v), 0, 0.25, causal)
    assert np.array_equal(o, ro.transpose(0, 2, 1, 3)) and np.array_equal(lse, rl)


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 3, 4, 8), dtype=np.uint16)
    k = np.zeros((1, 2, 4, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, k, k, 0, 1.0, False)  # Hq % Hkv != 0
    with pytest.raises(ValueError):
        oracle.attn_fwd(q[:, :2], k, k, 7, 1.0, False)  # unknown dtype
    sl = np.array([40], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.decode(np.zeros((1, 2, 8), np.uint16), np.zeros((1, 2, 32, 8), np.uint16),
                      np.zeros((1, 2, 32, 8), np.uint16), sl, 0, 1.0)  # L_b > max_len
