"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test names the passage it follows.  None of them re-types the oracle's
own loops: they use printed worked examples, closed forms, library routines
(numpy's float16 decoding, scipy's softmax / logsumexp), 40-digit decimal brute
force on tiny inputs, and invariances the pages claim.
"""
from decimal import Decimal, getcontext
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def contiguous_problem(q, k, v, scale=None, seq_lens=None):
    """q [B,Hq,d], k/v [B,N,Hkv,d] float32 -> (problem, args)."""
    B, Hq, d = q.shape
    _, N, Hkv, _ = k.shape
    p = oracle.problem(B, Hq, Hkv, d, "f32", N=N, scale=scale)
    return p, (q.astype(np.float32), k.astype(np.float32), v.astype(np.float32))


def scalar_row_problem(scores, vvals, d=64):
    """One request, one head, whose scaled scores are exactly `scores` and whose
    first V coordinate is `vvals` (all other coordinates 0).  q = 8 e0 with d = 64
    makes q.k / sqrt(64) = k0 exactly."""
    n = len(scores)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = math.sqrt(d)
    k = np.zeros((1, n, 1, d), np.float32)
    v = np.zeros((1, n, 1, d), np.float32)
    k[0, :, 0, 0] = scores
    v[0, :, 0, 0] = vvals
    return contiguous_problem(q, k, v)


getcontext().prec = 40


def brute_force(q, k, v, scale, lens=None, table=None, page=0):
    """40-digit decimal softmax attention straight from the definition."""
    B, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    sc = Decimal(1) / Decimal(d).sqrt() if scale is None else Decimal(float(scale))
    outs = np.zeros((B * Hq, d))
    lses = np.zeros(B * Hq)
    for b in range(B):
        n = k.shape[1] if lens is None else int(lens[b])
        for h in range(Hq):
            kvh = h // G
            rows = []
            for t in range(n):
                if page:
                    phys = table[b, t // page]
                    rows.append((k[phys, t % page, kvh], v[phys, t % page, kvh]))
                else:
                    rows.append((k[b, t, kvh], v[b, t, kvh]))
            s = [sum(Decimal(float(a)) * Decimal(float(c)) for a, c in zip(q[b, h], kr)) * sc for kr, _ in rows]
            m = max(s)
            w = [(x - m).exp() for x in s]
            Z = sum(w)
            for i in range(d):
                outs[b * Hq + h, i] = float(sum(wi * Decimal(float(vr[i])) for wi, (_, vr) in zip(w, rows)) / Z)
            lses[b * Hq + h] = float(m + Z.ln())
    return outs, lses


# ----------------------------------------------------------------------------
# storage decoding
# ----------------------------------------------------------------------------
def test_decode_f16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    got = oracle.decode(h, "f16")
    np.testing.assert_array_equal(got, h.astype(np.float64))


def test_decode_bf16_all_patterns_match_torch():
    """Every bfloat16 bit pattern against torch's own bfloat16 -> float64
    conversion (an implementation independent of the oracle and of synth)."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    # NaN: exponent all ones, mantissa non-zero (127 patterns per sign)
    assert int(nan.sum()) == 2 * 127
    np.testing.assert_array_equal(got[~nan], want[~nan])
    # signed zeros and infinities keep their sign; landmarks of the format
    assert got[0x0000] == 0.0 and math.copysign(1, got[0x8000]) < 0
    assert got[0x7F80] == np.inf and got[0xFF80] == -np.inf
    assert got[0x3F80] == 1.0 and got[0x4000] == 2.0 and got[0xC040] == -3.0
    assert got[0x0001] == 2.0 ** -133 and got[0x0080] == 2.0 ** -126


def test_decode_e4m3_all_patterns_match_torch_and_the_ocp_table():
    """8-bit cache values: OCP FP8 E4M3 (the handbook page's list of kernel
    improvements names FP8 KV caches converted in registers)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode(codes, "fp8")
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    np.testing.assert_array_equal(got[~nan], want[~nan])
    # the specification's landmarks: max normal S.1111.110 = 448, min normal
    # S.0001.000 = 2^-6, max subnormal S.0000.111 = 0.875 * 2^-6, min subnormal
    # S.0000.001 = 2^-9, one = S.0111.000
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x08] == 2.0 ** -6 and got[0x07] == 0.875 * 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x38] == 1.0 and got[0x00] == 0.0 and got[0x80] == 0.0 and math.copysign(1, got[0x80]) < 0


def _fp8_problem(rng, B, Hq, Hkv, d, N, k_scale, v_scale):
    q = synth.encode(rng.standard_normal((B, Hq, d)).astype(np.float32), "bf16")
    k = synth.encode(rng.standard_normal((B, N, Hkv, d)).astype(np.float32) * 40, "fp8")
    v = synth.encode(rng.standard_normal((B, N, Hkv, d)).astype(np.float32) * 40, "fp8")
    p = oracle.problem(B, Hq, Hkv, d, "fp8", N=N, q_dtype="bf16", k_scale=k_scale, v_scale=v_scale)
    return p, q, k, v


def test_brute_force_fp8_cache_with_scales():
    """A stored K or V value stands for stored * scale (one scale per tensor)."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, d, N = 1, 4, 2, 8, 7
    ks, vs = 0.037, 1.9
    p, q, k, v = _fp8_problem(rng, B, Hq, Hkv, d, N, ks, vs)
    out, lse = oracle.attention(p, q, k, v)
    dq = synth.decode_f64(q, "bf16")
    dk = synth.decode_f64(k, "fp8") * ks
    dv = synth.decode_f64(v, "fp8") * vs
    bo, bl = brute_force(dq, dk, dv, None)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_brute_force_fp8_cache_with_per_head_scales():
    """One scale per KV head (distinct, not powers of two): a stored value of
    KV head h stands for stored * scale[h], and query head j reads KV head
    j // G (the handbook's GQA map), so each query head sees its KV head's
    scales."""
    rng = np.random.default_rng(18)
    B, Hq, Hkv, d, N = 2, 6, 3, 8, 7
    ks = np.array([0.037, 0.51, 1.9])
    vs = np.array([1.9, 0.0071, 0.33])
    q = synth.encode(rng.standard_normal((B, Hq, d)).astype(np.float32), "bf16")
    k = synth.encode(rng.standard_normal((B, N, Hkv, d)).astype(np.float32) * 40, "fp8")
    v = synth.encode(rng.standard_normal((B, N, Hkv, d)).astype(np.float32) * 40, "fp8")
    p = oracle.problem(B, Hq, Hkv, d, "fp8", N=N, q_dtype="bf16", k_scales=ks, v_scales=vs)
    lens = np.array([7, 4], np.int32)
    out, lse = oracle.attention(p, q, k, v, seq_lens=lens)
    dk = synth.decode_f64(k, "fp8") * ks[None, None, :, None]
    dv = synth.decode_f64(v, "fp8") * vs[None, None, :, None]
    bo, bl = brute_force(synth.decode_f64(q, "bf16"), dk, dv, None, lens=lens)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)
    # the split partials merge to the same result
    po, pm, pl = oracle.split_partials(p, q, k, v, 3, 3, seq_lens=lens)
    mo, ml = oracle.merge(po, pm, pl)
    np.testing.assert_allclose(mo, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, bl, rtol=0, atol=1e-12)


def test_equal_per_head_scales_are_the_per_tensor_scale_bitwise():
    rng = np.random.default_rng(19)
    B, Hq, Hkv, d, N = 2, 8, 4, 16, 30
    c_k, c_v = 0.0377, 2.3
    p1, q, k, v = _fp8_problem(rng, B, Hq, Hkv, d, N, c_k, c_v)
    p2 = oracle.problem(B, Hq, Hkv, d, "fp8", N=N, q_dtype="bf16", k_scales=[c_k] * Hkv, v_scales=[c_v] * Hkv)
    for a, b in zip(oracle.attention(p1, q, k, v), oracle.attention(p2, q, k, v)):
        assert np.array_equal(a, b)


def test_a_kv_heads_scale_reaches_exactly_its_query_heads():
    """Changing the scales of KV head 1 changes the rows of query heads
    G .. 2G - 1 and no other row."""
    rng = np.random.default_rng(20)
    B, Hq, Hkv, d, N = 1, 8, 4, 16, 12
    _, q, k, v = _fp8_problem(rng, B, Hq, Hkv, d, N, 1.0, 1.0)
    base = np.array([0.5, 0.25, 0.125, 0.75])
    pa = oracle.problem(B, Hq, Hkv, d, "fp8", N=N, q_dtype="bf16", k_scales=base, v_scales=base)
    moved = base.copy()
    moved[1] = 0.3
    pb = oracle.problem(B, Hq, Hkv, d, "fp8", N=N, q_dtype="bf16", k_scales=moved, v_scales=moved)
    oa, la = oracle.attention(pa, q, k, v)
    ob, lb = oracle.attention(pb, q, k, v)
    G = Hq // Hkv
    changed = ~np.all(oa == ob, axis=1) | (la != lb)
    assert changed.tolist() == [G <= h < 2 * G for h in range(Hq)]


def test_per_head_scales_must_be_positive_and_finite():
    rng = np.random.default_rng(21)
    _, q, k, v = _fp8_problem(rng, 1, 4, 2, 8, 5, 1.0, 1.0)
    for bad in ([1.0, 0.0], [1.0, -2.0], [np.inf, 1.0], [np.nan, 1.0]):
        p = oracle.problem(1, 4, 2, 8, "fp8", N=5, q_dtype="bf16", k_scales=bad)
        with pytest.raises(ValueError):
            oracle.attention(p, q, k, v)


def test_fp8_cache_equals_the_fp32_cache_of_its_values_bitwise():
    """With power-of-two scales the dequantised values are exact fp32 numbers:
    the fp8 problem and the fp32 problem over those numbers agree bit for bit."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, N = 2, 8, 2, 16, 40
    p8, q, k, v = _fp8_problem(rng, B, Hq, Hkv, d, N, 2.0 ** -6, 2.0 ** 3)
    lens = np.array([40, 13], np.int32)
    o8, l8 = oracle.attention(p8, q, k, v, seq_lens=lens)
    q32 = synth.decode_f64(q, "bf16").astype(np.float32)
    k32 = (synth.decode_f64(k, "fp8") * 2.0 ** -6).astype(np.float32)
    v32 = (synth.decode_f64(v, "fp8") * 2.0 ** 3).astype(np.float32)
    p32 = oracle.problem(B, Hq, Hkv, d, "f32", N=N)
    o32, l32 = oracle.attention(p32, q32, k32, v32, seq_lens=lens)
    assert np.array_equal(o8, o32) and np.array_equal(l8, l32)
    # the same for the split partials
    a = oracle.split_partials(p8, q, k, v, 16, 3, seq_lens=lens)
    b = oracle.split_partials(p32, q32, k32, v32, 16, 3, seq_lens=lens)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ----------------------------------------------------------------------------
# several query tokens per request, causal (the handbook's FlashAttention
# forward kernel: query row i sees keys j <= i), new tokens at the end
# ----------------------------------------------------------------------------
def _multi_query_case(rng, B, q_len, Hq, Hkv, d, N, lens):
    q = rng.standard_normal((B, q_len, Hq, d)).astype(np.float32)
    k = rng.standard_normal((B, N, Hkv, d)).astype(np.float32) * 2
    v = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    p = oracle.problem(B, Hq, Hkv, d, "f32", N=N, q_len=q_len)
    return p, q, k, v, np.asarray(lens, np.int32)


def test_multi_query_brute_force_causal():
    rng = np.random.default_rng(21)
    B, L, Hq, Hkv, d, N = 2, 3, 2, 1, 4, 6
    p, q, k, v, lens = _multi_query_case(rng, B, L, Hq, Hkv, d, N, (6, 4))
    out, lse = oracle.attention(p, q, k, v, seq_lens=lens)
    for b in range(B):
        for i in range(L):
            n = int(lens[b]) - L + i + 1           # query i sits at position len - L + i
            bo, bl = brute_force(q[b:b + 1, i], k[b:b + 1, :n], v[b:b + 1, :n], None)
            r0 = (b * L + i) * Hq
            np.testing.assert_allclose(out[r0:r0 + Hq], bo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[r0:r0 + Hq], bl, rtol=0, atol=1e-12)


def test_multi_query_rows_are_single_queries_with_causal_lengths_bitwise():
    rng = np.random.default_rng(22)
    B, L, Hq, Hkv, d, N = 3, 4, 8, 2, 16, 50
    p, q, k, v, lens = _multi_query_case(rng, B, L, Hq, Hkv, d, N, (50, 9, 2))
    out, lse = oracle.attention(p, q, k, v, seq_lens=lens)
    po, pm, pl = oracle.split_partials(p, q, k, v, 8, 7, seq_lens=lens)
    for b in range(B):
        for i in range(L):
            n = max(0, int(lens[b]) - L + i + 1)
            p1 = oracle.problem(1, Hq, Hkv, d, "f32", N=N)
            o1, l1 = oracle.attention(p1, q[b, i][None], k[b:b + 1], v[b:b + 1], seq_lens=np.array([n], np.int32))
            a1, m1, s1 = oracle.split_partials(p1, q[b, i][None], k[b:b + 1], v[b:b + 1], 8, 7,
                                               seq_lens=np.array([n], np.int32))
            r = slice((b * L + i) * Hq, (b * L + i + 1) * Hq)
            assert np.array_equal(out[r], o1) and np.array_equal(lse[r], l1)
            assert np.array_equal(pm[r], m1) and np.array_equal(pl[r], s1)
            valid = s1 > 0
            assert np.array_equal(po[r][valid], a1[valid])
    # a query before the start of its request sees nothing
    r = (2 * L + 0) * Hq
    assert np.all(out[r:r + Hq] == 0.0) and np.all(lse[r:r + Hq] == -np.inf)


def test_prefill_equals_torch_causal_attention():
    """Every token of the request a query (q_len = len): the handbook's causal
    FlashAttention forward (page "FlashAttention and inference kernels",
    section "How FlashAttention evolved", the causal mask), which torch's
    scaled_dot_product_attention with is_causal computes (fp64, CPU); GQA by
    repeating each KV head for its group of consecutive query heads."""
    import torch
    rng = np.random.default_rng(31)
    B, L, Hq, Hkv, d = 2, 70, 8, 2, 16
    p, q, k, v, lens = _multi_query_case(rng, B, L, Hq, Hkv, d, L, (L, L))
    out, lse = oracle.attention(p, q, k, v, seq_lens=lens)
    G = Hq // Hkv
    tq = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)              # [B, Hq, L, d]
    tk = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    ref = ref.permute(0, 2, 1, 3).reshape(B * L * Hq, d).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_prefill_chunk_rows_equal_the_full_prefill_rows_bitwise():
    """A chunk of the last C query tokens (q_len = C) gives the rows of those
    tokens in a call with all L query tokens, bit for bit: the same keys per
    row, whatever the chunk's length (request 1 is shorter than L, so its
    first query tokens see nothing in the longer call)."""
    rng = np.random.default_rng(32)
    B, L, Hq, Hkv, d = 2, 45, 4, 4, 8
    pf, q, k, v, lens = _multi_query_case(rng, B, L, Hq, Hkv, d, L, (L, 30))
    full, lfull = oracle.attention(pf, q, k, v, seq_lens=lens)
    for C in (1, 7, 30):
        pc = oracle.problem(B, Hq, Hkv, d, "f32", N=L, q_len=C)
        qc = np.ascontiguousarray(q[:, L - C:])
        out, lse = oracle.attention(pc, qc, k, v, seq_lens=lens)
        for b in range(B):
            for i in range(C):
                # chunk query i and full query L - C + i both sit at position len - C + i
                rf = (b * L + L - C + i) * Hq
                rc = (b * C + i) * Hq
                assert np.array_equal(out[rc:rc + Hq], full[rf:rf + Hq]), (C, b, i)
                assert np.array_equal(lse[rc:rc + Hq], lfull[rf:rf + Hq]), (C, b, i)


# ----------------------------------------------------------------------------
# the handbook's worked online-softmax exercise
# ----------------------------------------------------------------------------
def test_worked_exercise_attention(golden):
    g = golden("handbook_online_softmax_exercise.json")
    p, (q, k, v) = scalar_row_problem(g["scores"], g["v"])
    out, lse = oracle.attention(p, q, k, v)
    assert abs(out[0, 0] - g["final"]) <= g["tol"]["final"]
    assert np.all(out[0, 1:] == 0.0)
    w = np.exp(np.array(g["scores"]))
    np.testing.assert_allclose(w, g["direct_weights"], atol=g["tol"]["direct_weights"])
    assert abs(w.sum() - g["direct_weight_sum"]) <= g["tol"]["direct_weight_sum"]
    assert abs(lse[0] - math.log(g["direct_weight_sum"])) < 1e-3


def test_worked_exercise_tile_trace(golden):
    g = golden("handbook_online_softmax_exercise.json")
    v = np.array(g["v"])[:, None]
    out, lse, tm, tl, ta = oracle.online_tiles(np.array(g["scores"]), v, g["tile"])
    tol = g["tol"]
    assert tm[0] == g["tile1"]["m"] and tm[1] == g["tile2"]["m"]
    assert abs(tl[0] - g["tile1"]["l"]) <= tol["l"]
    assert abs(tl[1] - g["tile2"]["l"]) <= tol["l"]
    assert abs(ta[0, 0] - g["tile1"]["acc"]) <= tol["acc"]
    assert abs(ta[1, 0] - g["tile2"]["acc"]) <= tol["acc"]
    assert abs(math.exp(g["tile1"]["m"] - g["tile2"]["m"]) - g["tile2"]["correction"]) <= tol["p"]
    assert abs(out[0] - g["final"]) <= tol["final"]


def test_worked_exercise_split_partials_and_merge(golden):
    """Split size 2 reproduces the two tiles as two splits (normalised O_s)."""
    g = golden("handbook_online_softmax_exercise.json")
    p, (q, k, v) = scalar_row_problem(g["scores"], g["v"])
    po, pm, pl = oracle.split_partials(p, q, k, v, split=2, S_max=2)
    assert pm[0, 0] == 3.0 and pm[0, 1] == 5.0
    assert abs(pl[0, 0] - g["tile1"]["l"]) <= g["tol"]["l"]
    # the page's first-tile accumulator is unnormalised: O_1 * l_1
    assert abs(po[0, 0, 0] * pl[0, 0] - g["tile1"]["acc"]) <= g["tol"]["acc"]
    assert abs(pl[0, 1] - sum(g["tile2"]["p"])) <= g["tol"]["p"] * 2
    for form in ("max", "lse"):
        out, lse = oracle.merge(po, pm, pl, form=form)
        assert abs(out[0, 0] - g["final"]) <= g["tol"]["final"]
    # merged denominator relative to the global max: the page's 1.2034
    lglob = pl[0, 0] * math.exp(pm[0, 0] - 5.0) + pl[0, 1]
    assert abs(lglob - g["tile2"]["l"]) <= g["tol"]["l"]


def test_worked_exercise_decimal_value():
    p, (q, k, v) = scalar_row_problem([1, 3, 2, 5], [10, 20, 30, 40])
    out, lse = oracle.attention(p, q, k, v)
    bo, bl = brute_force(q, k, v, None)
    assert abs(out[0, 0] - bo[0, 0]) < 1e-12 and abs(lse[0] - bl[0]) < 1e-12


# ----------------------------------------------------------------------------
# brute force on tiny inputs
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_contiguous(seed):
    rng = np.random.default_rng(100 + seed)
    B, Hq, Hkv, d, N = 2, 4, 2, 4, 6
    q = rng.standard_normal((B, Hq, d)).astype(np.float32) * 2
    k = rng.standard_normal((B, N, Hkv, d)).astype(np.float32) * 2
    v = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    lens = np.array([6, 3], np.int32)
    p, args = contiguous_problem(q, k, v)
    out, lse = oracle.attention(p, *args, seq_lens=lens)
    bo, bl = brute_force(q, k, v, None, lens=lens)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_brute_force_paged():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, d, page = 3, 4, 2, 4, 2
    lens = np.array([5, 1, 4], np.int32)
    nblk = (lens + page - 1) // page
    P = int(nblk.sum())
    perm = rng.permutation(P)
    table = np.full((B, 3), -1, np.int32)
    nx = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[nx:nx + nblk[b]]
        nx += nblk[b]
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    k = rng.standard_normal((P, page, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((P, page, Hkv, d)).astype(np.float32)
    p = oracle.problem(B, Hq, Hkv, d, "f32", page_size=page, max_blocks=3)
    out, lse = oracle.attention(p, q, k, v, seq_lens=lens, block_table=table)
    bo, bl = brute_force(q, k, v, None, lens=lens, table=table, page=page)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_brute_force_f16_and_bf16_storage():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, d, N = 1, 2, 1, 8, 5
    for dt in ("f16", "bf16"):
        qf = rng.standard_normal((B, Hq, d)).astype(np.float32)
        kf = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
        vf = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
        q, k, v = (synth.encode(x, dt) for x in (qf, kf, vf))
        p = oracle.problem(B, Hq, Hkv, d, dt, N=N)
        out, lse = oracle.attention(p, q, k, v)
        # the brute force reads the exactly decoded values
        dq, dk, dv = (synth.decode_f64(x, dt) for x in (q, k, v))
        bo, bl = brute_force(dq, dk, dv, None)
        np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_explicit_scale_argument():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 4)).astype(np.float32)
    k = rng.standard_normal((1, 4, 1, 4)).astype(np.float32)
    v = rng.standard_normal((1, 4, 1, 4)).astype(np.float32)
    p, args = contiguous_problem(q, k, v, scale=0.3)
    out, lse = oracle.attention(p, *args)
    bo, bl = brute_force(q, k, v, 0.3)
    np.testing.assert_allclose(out, bo, atol=1e-12)
    np.testing.assert_allclose(lse, bl, atol=1e-12)


# ----------------------------------------------------------------------------
# a special case that reduces to library routines
# ----------------------------------------------------------------------------
def test_identity_v_gives_scipy_softmax_and_logsumexp():
    """With V = I (d = N), the output row is the attention weight vector."""
    rng = np.random.default_rng(11)
    N = d = 16
    q = rng.standard_normal((1, 1, d)).astype(np.float32) * 3
    k = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    v = np.eye(N, dtype=np.float32).reshape(1, N, 1, d)
    p, args = contiguous_problem(q, k, v)
    out, lse = oracle.attention(p, *args)
    s = (k[0, :, 0, :].astype(np.float64) @ q[0, 0].astype(np.float64)) / math.sqrt(d)
    np.testing.assert_allclose(out[0], scipy.special.softmax(s), rtol=1e-13, atol=1e-15)
    assert abs(lse[0] - scipy.special.logsumexp(s)) < 1e-13


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def test_single_token_returns_its_value_row_bitwise():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 4, 8)).astype(np.float32)
    k = rng.standard_normal((2, 1, 2, 8)).astype(np.float32)
    v = rng.standard_normal((2, 1, 2, 8)).astype(np.float32)
    p, args = contiguous_problem(q, k, v)
    out, lse = oracle.attention(p, *args)
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[b * 4 + h], v[b, 0, h // 2].astype(np.float64))
            s = float(np.dot(q[b, h].astype(np.float64), k[b, 0, h // 2].astype(np.float64))) / math.sqrt(8)
            assert abs(lse[b * 4 + h] - s) < 1e-14


def test_identical_value_rows_return_that_row():
    rng = np.random.default_rng(2)
    N, d = 300, 16
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    k = rng.standard_normal((1, N, 1, d)).astype(np.float32) * 3
    row = rng.standard_normal(d).astype(np.float32)
    v = np.broadcast_to(row, (1, N, 1, d)).copy()
    p, args = contiguous_problem(q, k, v)
    out, _ = oracle.attention(p, *args)
    np.testing.assert_allclose(out, np.broadcast_to(row.astype(np.float64), (2, d)), rtol=1e-14, atol=1e-15)


def test_equal_scores_give_mean_of_v_and_log_n():
    rng = np.random.default_rng(3)
    N, d = 257, 8
    q = np.zeros((1, 1, d), np.float32)
    k = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    p, args = contiguous_problem(q, k, v)
    out, lse = oracle.attention(p, *args)
    np.testing.assert_allclose(out[0], v[0, :, 0, :].astype(np.float64).mean(axis=0), rtol=1e-13, atol=1e-15)
    assert lse[0] == math.log(N)


def test_shift_of_all_scores_leaves_output_and_shifts_lse():
    """k_t += (c sqrt(d) / |q|^2) q adds c to every scaled score."""
    rng = np.random.default_rng(4)
    N, d, c = 64, 16, 3.0
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, N, 1, d))
    v = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    alpha = c * math.sqrt(d) / float(q[0, 0] @ q[0, 0])
    # f32 storage rounds the shifted keys, so compare to the rounding level
    p, a0 = contiguous_problem(q.astype(np.float32), k.astype(np.float32), v)
    p1, a1 = contiguous_problem(q.astype(np.float32), (k + alpha * q[0, 0]).astype(np.float32), v)
    o0, l0 = oracle.attention(p, *a0)
    o1, l1 = oracle.attention(p1, *a1)
    np.testing.assert_allclose(o1, o0, atol=2e-5)
    assert abs(l1[0] - (l0[0] + c)) < 1e-4


def test_gqa_head_mapping_consecutive_heads_share_kv_head():
    """V of KV head j is the constant j + 1, so query head h must return h // G + 1."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, d, N = 2, 8, 2, 4, 10
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    k = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    v = np.zeros((B, N, Hkv, d), np.float32)
    for j in range(Hkv):
        v[:, :, j, :] = j + 1
    p, args = contiguous_problem(q, k, v)
    out, _ = oracle.attention(p, *args)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out[b * Hq + h], h // G + 1, rtol=1e-14)


def test_empty_request_gives_zero_and_minus_inf():
    q = np.ones((2, 1, 4), np.float32)
    k = np.ones((2, 3, 1, 4), np.float32)
    v = np.ones((2, 3, 1, 4), np.float32)
    p, args = contiguous_problem(q, k, v)
    out, lse = oracle.attention(p, *args, seq_lens=np.array([0, 3], np.int32))
    assert np.all(out[0] == 0) and lse[0] == -np.inf
    np.testing.assert_allclose(out[1], 1.0)


# ----------------------------------------------------------------------------
# paged indexing
# ----------------------------------------------------------------------------
def _paged_inputs(seed=0, page=16, lens=(1, 15, 16, 17, 255, 256, 257, 1000)):
    w = synth.with_lens(synth.Workload("t", B=1, Hq=4, Hkv=2, d=16, dtype="f32", split=32, N=16,
                                       page_size=page), lens)
    return synth.make_inputs(w, poison_tail=True)


def test_paged_equals_logically_contiguous_copy_bitwise():
    inp = _paged_inputs()
    w = inp.w
    p = oracle.problem_of(inp)
    out_p, lse_p = oracle.attention(p, inp.q, inp.k, inp.v, seq_lens=inp.seq_lens, block_table=inp.block_table)
    # gather into a contiguous [B, N, Hkv, d] cache in logical order
    kc = np.zeros((w.B, w.N, w.Hkv, w.d), np.float32)
    vc = np.zeros_like(kc)
    for b in range(w.B):
        for t in range(int(inp.seq_lens[b])):
            phys = inp.block_table[b, t // w.page_size]
            kc[b, t] = inp.k[phys, t % w.page_size]
            vc[b, t] = inp.v[phys, t % w.page_size]
    pc = oracle.problem(w.B, w.Hq, w.Hkv, w.d, "f32", N=w.N)
    out_c, lse_c = oracle.attention(pc, inp.q, kc, vc, seq_lens=inp.seq_lens)
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(lse_p, lse_c)
    assert np.isfinite(out_p).all()     # the NaN-poisoned tail slots were never read


def test_paged_probe_reads_the_page_formula_location():
    """V rows encode their physical (block, slot); one key per request is boosted so
    the softmax is one-hot on a chosen logical token t*.  The output names the
    physical row that the page's formula (slot t % page of block table[t / page])
    assigns to t*."""
    inp = _paged_inputs()
    w = inp.w
    P = inp.k.shape[0]
    k = np.zeros_like(inp.k)
    v = np.zeros_like(inp.v)
    for phys in range(P):
        for slot in range(w.page_size):
            v[phys, slot, :, 0] = phys
            v[phys, slot, :, 1] = slot
    q = np.zeros_like(inp.q)
    q[:, :, 0] = 1.0
    targets = []
    for b in range(w.B):
        n = int(inp.seq_lens[b])
        t_star = (7 * b + 3) % n
        phys = inp.block_table[b, t_star // w.page_size]
        k[phys, t_star % w.page_size, :, 0] = 400.0     # score 100 vs 0 elsewhere
        targets.append((phys, t_star % w.page_size))
    p = oracle.problem_of(inp)
    out, _ = oracle.attention(p, q, k, v, seq_lens=inp.seq_lens, block_table=inp.block_table)
    # every other weight is e^-100 relative, far below half an ulp of the result
    for b, (phys, slot) in enumerate(targets):
        for h in range(w.Hq):
            r = b * w.Hq + h
            assert out[r, 0] == phys and out[r, 1] == slot, (b, h, out[r, :2], phys, slot)


# ----------------------------------------------------------------------------
# split-KV: invariance to the split count and to the merge order
# ----------------------------------------------------------------------------
def _random_problem(seed=9, B=2, Hq=4, Hkv=2, d=8, N=100, lens=(100, 37)):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32) * 2
    k = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    p, args = contiguous_problem(q, k, v)
    return p, args, np.array(lens, np.int32)


@pytest.mark.parametrize("split", [1, 2, 3, 7, 16, 64, 100])
def test_split_count_invariance(split):
    p, args, lens = _random_problem()
    ref, lref = oracle.attention(p, *args, seq_lens=lens)
    S = -(-100 // split)
    po, pm, pl = oracle.split_partials(p, *args, split=split, S_max=S, seq_lens=lens)
    for form in ("max", "lse"):
        out, lse = oracle.merge(po, pm, pl, form=form)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lref, rtol=0, atol=1e-12)


def test_merge_order_invariance():
    p, args, lens = _random_problem()
    po, pm, pl = oracle.split_partials(p, *args, split=8, S_max=13, seq_lens=lens)
    o0, l0 = oracle.merge(po, pm, pl)
    perm = np.random.default_rng(1).permutation(13)
    o1, l1 = oracle.merge(po[:, perm], pm[:, perm], pl[:, perm])
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    np.testing.assert_allclose(l1, l0, atol=1e-13)


def test_partials_of_a_short_request_mark_empty_splits():
    p, args, lens = _random_problem()
    po, pm, pl = oracle.split_partials(p, *args, split=16, S_max=7, seq_lens=lens)
    # request 1 has 37 tokens -> splits 0..2 hold 16, 16, 5 tokens; 3..6 are empty
    Hq = p.Hq
    for h in range(Hq):
        r = Hq + h
        assert np.all(pl[r, :3] > 0) and np.all(pl[r, 3:] == 0)
        assert np.all(pm[r, 3:] == -np.inf)


def test_merge_skips_empty_splits_and_never_returns_nan():
    rng = np.random.default_rng(2)
    S, d = 5, 4
    po = rng.standard_normal((3, S, d))
    pm = rng.standard_normal((3, S))
    pl = rng.random((3, S)) + 0.5
    # row 0: two empty splits; row 1: all empty; row 2: untouched
    pm[0, [1, 3]] = -np.inf
    pl[0, [1, 3]] = 0.0
    po[0, [1, 3]] = np.nan         # an empty split's O must not be read
    pm[1] = -np.inf
    pl[1] = 0.0
    for form in ("max", "lse"):
        out, lse = oracle.merge(po, pm, pl, form=form)
        assert np.isfinite(out).all()
        ref0, lref0 = oracle.merge(po[:1, [0, 2, 4]], pm[:1, [0, 2, 4]], pl[:1, [0, 2, 4]], form=form)
        np.testing.assert_allclose(out[0], ref0[0], atol=1e-14)
        assert np.all(out[1] == 0) and lse[1] == -np.inf


def test_merge_forms_agree_with_a_direct_closed_form():
    """Two splits with known (m, l, O): the merge is the l e^m weighted mean."""
    po = np.array([[[1.0, 2.0], [3.0, -1.0]]])
    pm = np.array([[0.5, 2.0]])
    pl = np.array([[2.0, 0.25]])
    w = pl[0] * np.exp(pm[0])
    want = (w[:, None] * po[0]).sum(0) / w.sum()
    for form in ("max", "lse"):
        out, lse = oracle.merge(po, pm, pl, form=form)
        np.testing.assert_allclose(out[0], want, rtol=1e-15)
        assert abs(lse[0] - math.log(w.sum())) < 1e-14


# ----------------------------------------------------------------------------
# unified max value
# ----------------------------------------------------------------------------
def test_figure6_range_predicate(golden):
    g = golden("fdpp_figure6_range_check.json")
    lo, hi = g["phi"] + g["a"], g["phi"] + g["b"]
    for case in g["cases"]:
        sc = case["scores"]
        for s_idx, flag in enumerate(case["flagged_splits"]):
            part = sc[s_idx * g["split"]:(s_idx + 1) * g["split"]]
            assert any(oracle.out_of_range(x, lo, hi) for x in part) == bool(flag)


def test_figure6_through_unified_max(golden):
    g = golden("fdpp_figure6_range_check.json")
    lo, hi = g["phi"] + g["a"], g["phi"] + g["b"]
    for case in g["cases"]:
        p, (q, k, v) = scalar_row_problem(case["scores"], [1.0, 2.0, 3.0, 4.0])
        r = oracle.unified_max(p, q, k, v, split=2, S_max=2, phi=g["phi"], lo=lo, hi=hi)
        assert list(r["flags"][0]) == case["flagged_splits"]
        exact, else_ = oracle.attention(p, q, k, v)
        np.testing.assert_allclose(r["out"], exact, atol=1e-13)
        # unflagged splits keep phi; a flagged split uses its own max
        for s_idx, flag in enumerate(case["flagged_splits"]):
            part = case["scores"][2 * s_idx:2 * s_idx + 2]
            assert r["part_m"][0, s_idx] == (max(part) if flag else g["phi"])


def test_figure6_whole_row_fallback(golden):
    """The page's fallback recomputes the whole row: once a split of a row is
    flagged, every split of that row takes its own maximum.  Figure 6's
    second vector with y3 = 10 flags only the second half; its first half's
    own maximum (6) equals phi there, so the case is taken with y2 lowered to
    5 as well, where the first half's own maximum (5) differs from phi."""
    g = golden("fdpp_figure6_range_check.json")
    lo, hi = g["phi"] + g["a"], g["phi"] + g["b"]
    for scores_, want_m in [([3.0, 6.0, 10.0, 6.0], [6.0, 10.0]), ([3.0, 5.0, 10.0, 6.0], [5.0, 10.0])]:
        p, (q, k, v) = scalar_row_problem(scores_, [1.0, 2.0, 3.0, 4.0])
        split_r = oracle.unified_max(p, q, k, v, split=2, S_max=2, phi=g["phi"], lo=lo, hi=hi)
        row_r = oracle.unified_max(p, q, k, v, split=2, S_max=2, phi=g["phi"], lo=lo, hi=hi, whole_row=True)
        assert list(row_r["flags"][0]) == [0, 1] == list(split_r["flags"][0])
        assert list(row_r["part_m"][0]) == want_m
        assert list(split_r["part_m"][0]) == [g["phi"], 10.0]
        exact, lexact = oracle.attention(p, q, k, v)
        np.testing.assert_allclose(row_r["out"], exact, atol=1e-13)
        np.testing.assert_allclose(row_r["lse"], lexact, atol=1e-13)
    # the first vector stays in range: nothing is recomputed, phi everywhere
    p, (q, k, v) = scalar_row_problem([4.0, 5.0, 6.0, 7.0], [1.0, 2.0, 3.0, 4.0])
    r = oracle.unified_max(p, q, k, v, split=2, S_max=2, phi=g["phi"], lo=lo, hi=hi, whole_row=True)
    assert list(r["part_m"][0]) == [g["phi"], g["phi"]]


def test_whole_row_fallback_partials_are_the_synchronized_ones_bitwise():
    """A flagged row's partials are the synchronized split partials, bit for
    bit; an unflagged row's are those of the per-split fallback."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, d, N = 2, 4, 2, 16, 40
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    k = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    k[0, 7, 0] *= 12.0                   # one out-of-range score for the rows of KV head 0, request 0
    p, _ = contiguous_problem(q, k, v)
    lens = np.array([40, 23], np.int32)
    phi, lo, hi = -4.0, -4.0, 4.0
    kw = dict(split=8, S_max=5, phi=phi, lo=lo, hi=hi, seq_lens=lens)
    row_r = oracle.unified_max(p, q, k, v, whole_row=True, **kw)
    split_r = oracle.unified_max(p, q, k, v, **kw)
    so, sm, sl = oracle.split_partials(p, q, k, v, 8, 5, seq_lens=lens)
    row_flagged = row_r["flags"].any(axis=1)
    assert row_flagged.any() and not row_flagged.all()
    assert np.array_equal(row_r["flags"], split_r["flags"])
    for r in range(B * Hq):
        ref = (so, sm, sl) if row_flagged[r] else (split_r["part_o"], split_r["part_m"], split_r["part_l"])
        for got, want in zip((row_r["part_o"], row_r["part_m"], row_r["part_l"]), ref):
            assert np.array_equal(got[r], want[r]), r
    np.testing.assert_allclose(row_r["out"], split_r["out"], atol=1e-12)


@pytest.mark.parametrize("offset", [-40.0, -10.0, 0.0, 7.5, 40.0])
def test_unified_max_is_independent_of_phi(offset):
    p, args, lens = _random_problem(seed=12)
    exact, lexact = oracle.attention(p, *args, seq_lens=lens)
    phi = offset                   # scores are O(1): phi from far below to far above the max
    r = oracle.unified_max(p, *args, split=16, S_max=7, phi=phi, lo=-np.inf, hi=np.inf, seq_lens=lens)
    assert r["n_flagged"] == 0
    np.testing.assert_allclose(r["out"], exact, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["lse"], lexact, rtol=0, atol=1e-11)


def test_unified_max_all_flagged_equals_synchronized_partials_bitwise():
    p, args, lens = _random_problem(seed=13)
    sp_o, sp_m, sp_l = oracle.split_partials(p, *args, split=16, S_max=7, seq_lens=lens)
    r = oracle.unified_max(p, *args, split=16, S_max=7, phi=0.0, lo=1e30, hi=1e31, seq_lens=lens)
    valid = sp_l > 0
    assert r["n_flagged"] == int(valid.sum())
    np.testing.assert_array_equal(r["flags"].astype(bool), valid)
    np.testing.assert_array_equal(r["part_m"], sp_m)
    np.testing.assert_array_equal(r["part_l"], sp_l)
    np.testing.assert_array_equal(r["part_o"], sp_o)


def test_unified_max_flag_rate_matches_closed_form():
    """Stress recipe: key rows scaled x8 with probability 0.02.  For a fixed q, a
    clean score is N(0, |q|^2/d) and a stressed one N(0, 64|q|^2/d); a split of L
    tokens is flagged with probability 1 - (1 - p_tok)^L where p_tok is the
    two-sided tail beyond [-c, c] of that mixture."""
    w = synth.Workload("stress_small", B=2, Hq=16, Hkv=16, d=128, dtype="bf16", split=256, N=4096,
                       stress_frac=0.02, stress_scale=8.0)
    inp = synth.make_inputs(w)
    p = oracle.problem_of(inp)
    c = 12.0
    r = oracle.unified_max(p, inp.q, inp.k, inp.v, split=w.split, S_max=w.max_splits, phi=-c, lo=-c, hi=c)
    qf = synth.decode_f64(inp.q, w.dtype)
    sig = np.linalg.norm(qf, axis=-1).reshape(-1) / math.sqrt(w.d)
    tail = lambda x: math.erfc(x / math.sqrt(2.0))      # P(|Z| > x)
    expected = 0.0
    var = 0.0
    for s in sig:
        pt = 0.98 * tail(c / s) + 0.02 * tail(c / (8 * s))
        ps = 1 - (1 - pt) ** w.split
        expected += ps * w.max_splits
        var += ps * (1 - ps) * w.max_splits
    got = r["n_flagged"]
    assert abs(got - expected) < 5 * math.sqrt(var) + 1, (got, expected, var)
    assert 0.2 < got / (sig.size * w.max_splits) < 0.8      # the closed form puts it near one half
    # and the fallback keeps the result exact
    exact, _ = oracle.attention(p, inp.q, inp.k, inp.v)
    np.testing.assert_allclose(r["out"], exact, rtol=1e-10, atol=1e-12)


def test_oracle_rejects_bad_shapes():
    q = np.zeros((1, 3, 4), np.float32)
    k = np.zeros((1, 2, 2, 4), np.float32)
    p = oracle.problem(1, 3, 2, 4, "f32", N=2)       # Hq not a multiple of Hkv
    with pytest.raises(ValueError):
        oracle.attention(p, q, k, k)
