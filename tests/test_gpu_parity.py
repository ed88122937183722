"""GPU parity of the split-KV decode-attention library against the fp64 oracle.

Every case runs the HIP kernels through the C ABI on seeded synth inputs and
compares element by element with the oracle on the same inputs, at the bar
stated in fdtest.py.  The five workload shapes run at full size, every query
row compared (out, lse and the split partials); smaller
cases cover the edges: ragged and empty requests, every dtype, head
dimension and group size, split sizes from 1 token to a single split, page
sizes from 1 to 64 tokens, poisoned cache tails, invalid page entries, caches
addressed beyond 4 GiB, both launch regimes of the MFMA kernel, 8-bit caches,
several query tokens per request, and the unified-max fallback.
"""
import dataclasses
import math

import numpy as np
import pytest

import fdtest as ft
from fdtest import Run, say
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = ft.torch()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_attn_amd as fd
    fd.lib()


KERNELS = ["valu", "mfma"]


def _kernel_ok(kernel, dtype):
    return kernel == "valu" or dtype in ("f16", "bf16")


def _skip_unsupported(fn):
    """Run fn(); skip the case when the library reports the kernel unsupported."""
    import decode_attention_attn_amd as fd
    try:
        return fn()
    except fd.FdError as e:
        if e.status == fd.FD_ERR_UNSUPPORTED:
            pytest.skip("kernel not available for this shape")
        raise


# ----------------------------------------------------------------------------
# the handbook's worked exercise, on the GPU
# ----------------------------------------------------------------------------
def test_worked_exercise(golden):
    g = golden("handbook_online_softmax_exercise.json")
    d, n = 64, 4
    w = synth.Workload("exercise", B=1, Hq=1, Hkv=1, d=d, dtype="f32", split=2, N=n)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = math.sqrt(d)        # q.k / sqrt(d) = k0
    k = np.zeros((1, n, 1, d), np.float32)
    v = np.zeros((1, n, 1, d), np.float32)
    k[0, :, 0, 0] = g["scores"]
    v[0, :, 0, 0] = g["v"]
    inp = synth.Inputs(w, q, k, v, np.array([n], np.int32))
    res = Run(inp).run()
    say(f"exercise: out[0]={res['out'][0, 0]!r}")
    assert abs(res["out"][0, 0] - g["final"]) <= g["tol"]["final"]
    ft.check_exact(res, inp, what="exercise")
    # the two splits are the page's two tiles
    assert res["part_m"][0].tolist() == [3.0, 5.0]
    assert abs(res["part_l"][0, 0] - g["tile1"]["l"]) <= g["tol"]["l"]
    assert abs(res["part_o"][0, 0, 0] * res["part_l"][0, 0] - g["tile1"]["acc"]) <= g["tol"]["acc"]


# ----------------------------------------------------------------------------
# the workload shapes at full size
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_mha", "llama2_7b_mha", "long_gqa_32k"])
def test_workload_full(name):
    w = synth.WORKLOADS[name]
    say(f"[{name}] generating")
    inp = synth.make_inputs(w)
    r = Run(inp)
    res = r.run()
    e1, e2 = ft.check_exact(res, inp, what=name)
    ft.check_partials(res, inp, w.split, what=name)
    say(f"[{name}] max|out err|={e1:.3e} max|lse err|={e2:.3e}")
    # the same kernels without a seq_lens array (every request full length)
    res2 = r.run(use_lens=False)
    assert np.array_equal(res2["out"], res["out"]) and np.array_equal(res2["lse"], res["lse"])


def test_paged_batched_gqa_full():
    w = synth.WORKLOADS["paged_batched_gqa"]
    say("[paged_batched_gqa] generating")
    inp = synth.make_inputs(w)
    say(f"[paged_batched_gqa] {inp.k.shape[0]} pages, kv bytes {inp.kv_bytes}")
    r = Run(inp)
    # the separate merge keeps the split partials in the workspace; AUTO takes
    # the single launch for this shape (its partial rows are then internal)
    res = r.run(merge="separate")
    auto = r.run()
    assert np.isfinite(res["out"]).all() and np.isfinite(res["lse"]).all()
    say("[paged_batched_gqa] GPU done; oracle on every row")
    ref, lref = ft.oracle_exact(inp)
    for what, x in (("separate", res), ("auto", auto)):
        e1 = ft.assert_close(x["out"], ref, w.dtype, f"paged_batched_gqa {what} out")
        e2 = ft.assert_close(x["lse"], lref, w.dtype, f"paged_batched_gqa {what} lse")
        say(f"[paged_batched_gqa] {what}, all {len(x['lse'])} rows: max|out err|={e1:.3e} max|lse err|={e2:.3e}")
    ft.check_partials(res, inp, w.split, what="paged_batched_gqa")


def _stress_rate_expectation(inp, c):
    """Closed-form expected number of flagged (row, split) pairs for bounds [-c, c]."""
    w = inp.w
    qf = synth.decode_f64(inp.q, w.dtype)
    sig = np.linalg.norm(qf, axis=-1).reshape(-1) / math.sqrt(w.d)
    tail = lambda x: math.erfc(x / math.sqrt(2.0))
    exp_count = 0.0
    for s in sig:
        pt = (1 - w.stress_frac) * tail(c / s) + w.stress_frac * tail(c / (w.stress_scale * s))
        exp_count += (1 - (1 - pt) ** w.split) * w.max_splits
    return exp_count


def test_umax_stress_full():
    """Every row of the stress shape against the oracle: the synchronized path
    (out, lse, split partials), and both unified-max bound sets (out, lse, the
    flag set, and the partials of every split whose flag agrees with the
    oracle's: phi-scaled where unflagged, recomputed where flagged)."""
    import oracle
    w = synth.WORKLOADS["umax_stress"]
    say("[umax_stress] generating")
    inp = synth.make_inputs(w)
    r = Run(inp)
    sync = r.run()
    say("[umax_stress] sync done; oracle on every row")
    ref, lref = ft.oracle_exact(inp)
    ft.assert_close(sync["out"], ref, w.dtype, "umax_stress sync out")
    ft.assert_close(sync["lse"], lref, w.dtype, "umax_stress sync lse")
    ft.check_partials(sync, inp, w.split, what="umax_stress sync")
    R, S = w.B * w.Hq, w.max_splits
    p = oracle.problem_of(inp)
    for phi, lo, hi in [(-6.0, -6.0, 6.0), (-20.0, -20.0, 20.0)]:
        res = r.run(mode="unified", phi=phi, lo=lo, hi=hi)
        nflag = int(res["flags"].sum())
        rate = nflag / (R * S)
        expect = _stress_rate_expectation(inp, hi) / (R * S)
        say(f"[umax_stress] bounds [{lo}, {hi}] phi={phi}: fallback rate {rate:.4f} (closed form {expect:.4f})")
        assert set(np.unique(res["flags"])) <= {0, 1}
        assert res["count"] == nflag
        assert abs(rate - expect) < 0.05 + 0.1 * expect
        ft.assert_close(res["out"], ref, w.dtype, f"umax_stress unified {hi} out")
        ft.assert_close(res["lse"], lref, w.dtype, f"umax_stress unified {hi} lse")
        must, may = ft.flag_bounds(inp, w.split, S, phi, lo, hi)
        got = res["flags"].astype(bool)
        assert np.all(got[must]), "a split with a clearly out-of-range score was not flagged"
        assert not np.any(got[~may]), "a split with only in-range scores was flagged"
        uo = oracle.unified_max(p, inp.q, inp.k, inp.v, w.split, S, phi, lo, hi, seq_lens=inp.seq_lens)
        agree = (uo["flags"].astype(bool) == got) & (uo["part_l"] > 0)
        say(f"[umax_stress] {int(agree.sum())} of {agree.size} splits compared")
        for key in ("part_m", "part_l", "part_o"):
            ft.assert_close(res[key][agree], uo[key][agree], w.dtype, f"umax_stress unified {hi} {key}")


# ----------------------------------------------------------------------------
# dtype x head dim x group size x kernel on ragged requests
# ----------------------------------------------------------------------------
# G = 1, 2, 3, 8, 16, and 3 with an odd KV head count (whose resident grids keep grid-order heads;
# even counts take the odd heads first)
GROUPS = [(8, 8), (8, 4), (12, 4), (16, 2), (32, 2), (9, 3)]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", GROUPS)
def test_shapes(kernel, dtype, d, Hq, Hkv):
    if not _kernel_ok(kernel, dtype):
        pytest.skip("mfma kernel is 16-bit only")
    base = synth.Workload("shape", B=3, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, split=128, N=1)
    inp = synth.make_inputs(synth.with_lens(base, (1000, 1, 385)))
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel))
    ft.check_exact(res, inp, what=f"{kernel} {dtype} d={d} G={Hq // Hkv}")
    ft.check_partials(res, inp, 128, what=f"{kernel} {dtype} d={d} G={Hq // Hkv}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("split", [1, 16, 100, 256, 512, 5000])
def test_split_sizes(kernel, split):
    base = synth.Workload("splits", B=2, Hq=16, Hkv=4, d=128, dtype="bf16", split=split, N=1)
    inp = synth.make_inputs(synth.with_lens(base, (4096, 777)))
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel, split=split))
    ft.check_exact(res, inp, what=f"split {split}")
    ft.check_partials(res, inp, split, what=f"split {split}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("page", [0, 16])
def test_awkward_lengths(kernel, page):
    lens = (1, 15, 16, 17, 255, 256, 257, 1000, 4096)
    base = synth.Workload("lens", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", split=256, N=1, page_size=page)
    inp = synth.make_inputs(synth.with_lens(base, lens))
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel))
    ft.check_exact(res, inp, what=f"lengths page={page}")
    ft.check_partials(res, inp, 256, what=f"lengths page={page}")


# both launch regimes of the MFMA kernel on a 16-bit cache: one wave per
# workgroup from four workgroups per CU, two below; workgroups = splits of
# the longest request x KV heads x requests, split 256, 256 CUs
REGIMES = [
    (16, 16, (4096, 3000)),                   # G=1, 512 workgroups: two waves
    (16, 16, (4096,) * 6 + (3001, 17)),       # G=1, 2048: one
    (32, 8, (4096, 2900, 1)),                 # G=4, 384: two
    (32, 8, (4096,) * 7 + (100,)),            # G=4, 1024: one
    (64, 8, (4096,) * 3 + (2500,)),           # G=8, 512: two
    (64, 8, (4096,) * 8 + (2500,)),           # G=8, 1152: one
]


@pytest.mark.parametrize("page", [0, 16])
@pytest.mark.parametrize("mode", ["sync", "unified"])
@pytest.mark.parametrize("Hq,Hkv,lens", REGIMES)
def test_launch_regimes(Hq, Hkv, lens, mode, page):
    base = synth.Workload("regime", B=1, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", split=256, N=1, page_size=page,
                          stress_frac=0.02, stress_scale=8.0)
    inp = synth.make_inputs(synth.with_lens(base, lens))
    what = f"G={Hq // Hkv} B={len(lens)} {mode} page={page}"
    say(f"[regime] {what}")
    if mode == "sync":
        res = Run(inp).run(kernel="mfma")
        ft.check_partials(res, inp, 256, what=what)
    else:
        res = Run(inp).run(kernel="mfma", mode="unified", phi=-12.0, lo=-12.0, hi=12.0)
        assert res["count"] == int(res["flags"].sum()) and 0 < res["count"] < res["flags"].size
    ft.check_exact(res, inp, what=what)


@pytest.mark.parametrize("page", [0, 16])
def test_empty_request_gives_zero_and_minus_inf(page):
    base = synth.Workload("empty", B=3, Hq=8, Hkv=2, d=128, dtype="bf16", split=64, N=1, page_size=page)
    inp = synth.make_inputs(synth.with_lens(base, (0, 100, 0)))
    res = Run(inp).run()
    for b in (0, 2):
        rows = slice(b * 8, (b + 1) * 8)
        assert np.all(res["out"][rows] == 0.0)
        assert np.all(res["lse"][rows] == -np.inf)
    ft.check_exact(res, inp, rows=np.arange(8, 16), what=f"empty page={page}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_token_returns_its_value_row_bitwise(dtype):
    base = synth.Workload("one", B=2, Hq=8, Hkv=4, d=128, dtype=dtype, split=256, N=1)
    inp = synth.make_inputs(synth.with_lens(base, (1, 1)))
    res = Run(inp).run()
    raw = res["raw_out"].reshape(2, 8, 128)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(raw[b, h], inp.v[b, 0, h // 2]), (b, h)


def test_equal_scores_give_mean_of_v_and_log_n():
    base = synth.Workload("q0", B=1, Hq=4, Hkv=1, d=128, dtype="f32", split=256, N=1000)
    inp = synth.make_inputs(base)
    inp.q[:] = 0
    res = Run(inp).run()
    mean = inp.v[0, :, 0, :].astype(np.float64).mean(axis=0)
    for h in range(4):
        ft.assert_close(res["out"][h], mean, "f32", "mean of V")
        ft.assert_close(res["lse"][h], math.log(1000), "f32", "ln N")


def test_identical_value_rows():
    base = synth.Workload("vrow", B=1, Hq=8, Hkv=2, d=128, dtype="bf16", split=256, N=3000)
    inp = synth.make_inputs(base)
    inp.v[:] = inp.v[0, 0]
    res = Run(inp).run()
    for h in range(8):
        want = synth.decode_f64(inp.v[0, 0, h // 4], "bf16")
        ft.assert_close(res["out"][h], want, "bf16", "identical V rows")


def test_out_dtype_can_differ_from_cache_dtype():
    base = synth.Workload("outf32", B=2, Hq=16, Hkv=4, d=128, dtype="bf16", split=128, N=700)
    inp = synth.make_inputs(base)
    res = Run(inp).run(out_dtype="f32")
    ft.check_exact(res, inp, what="f32 out from bf16 cache")


# ----------------------------------------------------------------------------
# paged indexing: bit-exact
# ----------------------------------------------------------------------------
def _relabel_pages(inp, new_table_of):
    """Same logical data under another physical assignment: returns a new Inputs."""
    w = inp.w
    P = inp.k.shape[0]
    new_table = new_table_of(inp.block_table, P)
    k = np.empty_like(inp.k)
    v = np.empty_like(inp.v)
    valid = inp.block_table >= 0
    k[new_table[valid]] = inp.k[inp.block_table[valid]]
    v[new_table[valid]] = inp.v[inp.block_table[valid]]
    return synth.Inputs(w, inp.q, k, v, inp.seq_lens, new_table)


@pytest.mark.parametrize("kernel", KERNELS)
def test_paged_permutation_is_bitwise_invariant(kernel):
    base = synth.Workload("perm", B=4, Hq=32, Hkv=8, d=128, dtype="bf16", split=256, N=1, page_size=16)
    inp = synth.make_inputs(synth.with_lens(base, (3000, 17, 1024, 4100)))

    def identity(table, P):
        t = np.full_like(table, -1)
        nxt = 0
        for b in range(table.shape[0]):
            n = int((table[b] >= 0).sum())
            t[b, :n] = np.arange(nxt, nxt + n)
            nxt += n
        return t

    def reversed_(table, P):
        t = table.copy()
        t[table >= 0] = P - 1 - table[table >= 0]
        return t

    r0 = _skip_unsupported(lambda: Run(inp).run(kernel=kernel))
    for relabel in (identity, reversed_):
        r1 = Run(_relabel_pages(inp, relabel)).run(kernel=kernel)
        for key in ("out", "lse", "part_o", "part_m", "part_l"):
            a, b = r0[key], r1[key]
            if key == "part_o":      # O rows of empty splits are unwritten
                a, b = a[r0["part_l"] > 0], b[r0["part_l"] > 0]
            assert np.array_equal(a, b), (relabel.__name__, key)
    ft.check_exact(r0, inp, what="perm")


@pytest.mark.parametrize("kernel", ["auto"] + KERNELS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page", [1, 8, 32, 64])
def test_page_sizes(page, d, kernel):
    """Pages of 1 to 64 tokens: the MFMA kernel takes pages of a multiple of
    16 tokens and reports the others unsupported; auto falls back to the VALU
    kernel there."""
    import decode_attention_attn_amd as fd
    base = synth.Workload("pages", B=3, Hq=16, Hkv=4, d=d, dtype="bf16", split=256, N=1, page_size=page)
    inp = synth.make_inputs(synth.with_lens(base, (1000, 257, 2048)))
    what = f"page={page} d={d} {kernel}"
    if kernel == "mfma" and page % 16:
        with pytest.raises(fd.FdError) as e:
            Run(inp).run(kernel=kernel)
        assert e.value.status == fd.FD_ERR_UNSUPPORTED
        return
    res = Run(inp).run(kernel=kernel)
    ft.check_exact(res, inp, what=what)
    ft.check_partials(res, inp, 256, what=what)


@pytest.mark.parametrize("kernel", KERNELS)
def test_paged_pool_beyond_4_gib(kernel):
    """The requests' pages sit at the top of a pool of 4.3 GiB per cache (byte
    offsets past 2^32); the rest of the pool is never written and must never
    be read.  Same bits as the compact pool, and the oracle's values."""
    t = ft.torch()
    base = synth.Workload("bigpool", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", split=256, N=1, page_size=16)
    inp = synth.make_inputs(synth.with_lens(base, (3000, 1500)))
    small = Run(inp).run(kernel=kernel)
    P = inp.k.shape[0]
    P_big = 140_000                                   # 140000 pages of 32 KiB: 4.27 GiB per cache
    shift = P_big - P
    r = Run(inp)
    big_k = t.empty((P_big,) + tuple(r.k.shape[1:]), dtype=r.k.dtype, device="cuda")
    big_v = t.empty_like(big_k)
    big_k[shift:] = r.k
    big_v[shift:] = r.v
    table = inp.block_table.copy()
    table[table >= 0] += shift
    r.k, r.v = big_k, big_v
    r.table = t.from_numpy(table).to("cuda")
    res = r.run(kernel=kernel)
    for key in ("out", "lse", "part_m", "part_l"):
        assert np.array_equal(res[key], small[key]), key
    ft.check_exact(res, inp, what=f"pool beyond 4 GiB {kernel}")
    del big_k, big_v
    t.cuda.empty_cache()


@pytest.mark.parametrize("kernel", KERNELS)
def test_contiguous_cache_beyond_4_gib(kernel):
    """Request 1 of a contiguous cache with 2^21 tokens of capacity starts
    4 GiB into each cache; only the first len tokens of each request are
    written.  Same bits as a cache of capacity N, and the oracle's values."""
    import decode_attention_attn_amd as fd
    t = ft.torch()
    base = synth.Workload("bigcache", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", split=256, N=1)
    inp = synth.make_inputs(synth.with_lens(base, (3000, 1500)))
    w = inp.w
    r = Run(inp)
    small = r.run(kernel=kernel)
    cap = 1 << 21                                     # 2^21 tokens x 2 KiB = 4 GiB per request
    big_k = t.empty((w.B, cap, w.Hkv, w.d), dtype=r.k.dtype, device="cuda")
    big_v = t.empty_like(big_k)
    for b in range(w.B):
        n = int(inp.seq_lens[b])
        big_k[b, :n] = r.k[b, :n]
        big_v[b, :n] = r.v[b, :n]
    desc = r.desc(kernel=kernel)
    po, pm, pl, _ = fd.alloc_partials(desc)
    out = t.empty((w.B, w.Hq, w.d), dtype=t.bfloat16, device="cuda")
    lse = t.empty((w.B, w.Hq), dtype=t.float32, device="cuda")
    fd.fd_decode_attn_partial(desc, r.q, big_k, big_v, cap, r.lens, po, pm, pl)
    fd.fd_decode_attn_combine(desc, po, pm, pl, r.lens, out, lse)
    t.cuda.synchronize()
    R = w.B * w.Hq
    got_out, got_lse = ft.f64(out).reshape(R, w.d), ft.f64(lse).reshape(R)
    assert np.array_equal(got_out, small["out"]) and np.array_equal(got_lse, small["lse"])
    ft.check_exact(dict(out=got_out, lse=got_lse), inp, what=f"cache beyond 4 GiB {kernel}")
    del big_k, big_v
    t.cuda.empty_cache()


def test_paged_probe_reads_the_page_formula_location():
    """V rows encode their physical (block, slot) and one key per request is
    boosted so the softmax is one-hot; the output names the physical row."""
    base = synth.Workload("probe", B=5, Hq=8, Hkv=2, d=128, dtype="f32", split=64, N=1, page_size=16)
    inp = synth.make_inputs(synth.with_lens(base, (1, 33, 300, 16, 1000)))
    w = inp.w
    P = inp.k.shape[0]
    inp.k[:] = 0
    inp.q[:] = 0
    inp.q[:, :, 0] = 1.0
    for phys in range(P):
        for slot in range(16):
            inp.v[phys, slot, :, 0] = phys
            inp.v[phys, slot, :, 1] = slot
    targets = []
    for b in range(w.B):
        n = int(inp.seq_lens[b])
        t_star = (7 * b + 3) % n
        phys = inp.block_table[b, t_star // 16]
        inp.k[phys, t_star % 16, :, 0] = 800.0       # score 800 / sqrt(128) ~ 70.7 vs 0
        targets.append((phys, t_star % 16))
    res = Run(inp).run()
    for b, (phys, slot) in enumerate(targets):
        for h in range(w.Hq):
            r = b * w.Hq + h
            assert res["out"][r, 0] == phys and res["out"][r, 1] == slot, (b, h, res["out"][r, :2])


def test_invalid_page_entries_are_not_read():
    """A block-table entry outside the pool makes its 16 tokens absent."""
    base = synth.Workload("badpage", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", split=64, N=1, page_size=16)
    inp = synth.make_inputs(synth.with_lens(base, (160, 64)))
    bad = inp.block_table.copy()
    bad[0, 3] = -1
    bad[1, 1] = 10 ** 6
    binp = synth.Inputs(inp.w, inp.q, inp.k, inp.v, inp.seq_lens, bad)
    res = Run(binp).run()
    # expected: the same requests with those pages' tokens removed
    keep0 = [t for t in range(160) if t // 16 != 3]
    keep1 = [t for t in range(64) if t // 16 != 1]
    n = max(len(keep0), len(keep1))
    wc = synth.Workload("badpage_ref", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", split=64, N=n)
    kc = np.zeros((2, n, 2, 128), np.uint16)
    vc = np.zeros_like(kc)
    for b, keep in enumerate((keep0, keep1)):
        for i, t in enumerate(keep):
            kc[b, i] = inp.k[inp.block_table[b, t // 16], t % 16]
            vc[b, i] = inp.v[inp.block_table[b, t // 16], t % 16]
    ref_inp = synth.Inputs(wc, inp.q, kc, vc, np.array([len(keep0), len(keep1)], np.int32))
    ref, lref = ft.oracle_exact(ref_inp)
    ft.assert_close(res["out"], ref, "bf16", "invalid pages out")
    ft.assert_close(res["lse"], lref, "bf16", "invalid pages lse")


def test_repeat_runs_are_bitwise_identical():
    base = synth.Workload("repeat", B=2, Hq=64, Hkv=8, d=128, dtype="bf16", split=256, N=1, page_size=16)
    inp = synth.make_inputs(synth.with_lens(base, (5000, 2049)))
    r = Run(inp)
    a = r.run()
    b = r.run()
    for key in ("out", "lse", "part_m", "part_l"):
        assert np.array_equal(a[key], b[key]), key


# ----------------------------------------------------------------------------
# unified max value
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("page", [0, 16])
def test_unified_max_flags_and_fallback(kernel, page):
    base = synth.Workload("umax", B=2, Hq=32, Hkv=4, d=128, dtype="bf16", split=256, N=1, page_size=page,
                          stress_frac=0.02, stress_scale=8.0)
    inp = synth.make_inputs(synth.with_lens(base, (4096, 1500)))
    w = inp.w
    S = -(-w.N // w.split)
    phi, lo, hi = -12.0, -12.0, 12.0
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel, mode="unified", phi=phi, lo=lo, hi=hi))
    must, may = ft.flag_bounds(inp, w.split, S, phi, lo, hi)
    got = res["flags"].astype(bool)
    assert np.all(got[must]) and not np.any(got[~may])
    assert res["count"] == int(got.sum()) and 0 < got.sum() < got.size
    ft.check_exact(res, inp, what="unified")
    # partials: unflagged splits use phi, flagged ones their own maximum
    import oracle
    p = oracle.problem_of(inp)
    uo = oracle.unified_max(p, inp.q, inp.k, inp.v, w.split, S, phi, lo, hi, seq_lens=inp.seq_lens,
                            block_table=inp.block_table)
    agree = (uo["flags"].astype(bool) == got) & (uo["part_l"] > 0)
    for key in ("part_m", "part_l", "part_o"):
        ft.assert_close(res[key][agree], uo[key][agree], "bf16", f"unified {key}")


@pytest.mark.parametrize("page", [0, 16])
@pytest.mark.parametrize("kernel", KERNELS)
def test_unified_max_whole_row_fallback(kernel, page):
    """FD_FALLBACK_ROW: a query row with any flagged split has all of its
    splits recomputed synchronized (the FlashDecoding++ page's whole-row
    fallback).  Its partials are then bit for bit those of the synchronized
    path, an unflagged row's those of the per-split fallback (which leaves it
    alone too); the flags are the same in both modes; out and lse match the
    oracle, and so do the partials against the oracle's whole-row fallback
    wherever the GPU and the oracle flag a row alike."""
    import oracle
    base = synth.Workload("umaxrow", B=2, Hq=32, Hkv=4, d=128, dtype="bf16", split=256, N=1, page_size=page,
                          stress_frac=0.02, stress_scale=8.0)
    inp = synth.make_inputs(synth.with_lens(base, (4096, 1500)))
    w = inp.w
    S = -(-w.N // w.split)
    phi, lo, hi = -16.0, -16.0, 16.0
    r = Run(inp)
    row = _skip_unsupported(lambda: r.run(kernel=kernel, mode="unified", phi=phi, lo=lo, hi=hi, fallback="row"))
    split = r.run(kernel=kernel, mode="unified", phi=phi, lo=lo, hi=hi)
    sync = r.run(kernel=kernel)
    assert np.array_equal(row["flags"], split["flags"]) and row["count"] == split["count"]
    rows_flagged = row["flags"].astype(bool).any(axis=1)
    assert rows_flagged.any() and not rows_flagged.all()
    valid = sync["part_l"] > 0
    for key in ("part_m", "part_l", "part_o"):
        a, b_sync, b_split = row[key], sync[key], split[key]
        for rr in range(a.shape[0]):
            v = valid[rr]
            want = b_sync[rr][v] if rows_flagged[rr] else b_split[rr][v]
            assert np.array_equal(a[rr][v], want), (key, rr, bool(rows_flagged[rr]))
    ft.check_exact(row, inp, what=f"whole-row fallback {kernel} page={page}")
    uo = oracle.unified_max(oracle.problem_of(inp), inp.q, inp.k, inp.v, w.split, S, phi, lo, hi,
                            seq_lens=inp.seq_lens, block_table=inp.block_table, whole_row=True)
    agree = (uo["flags"].astype(bool).any(axis=1) == rows_flagged)[:, None] & (uo["part_l"] > 0)
    for key in ("part_m", "part_l", "part_o"):
        ft.assert_close(row[key][agree], uo[key][agree], "bf16", f"whole-row {key}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_unified_max_all_flagged_is_bitwise_the_synchronized_path(kernel):
    base = synth.Workload("umax_all", B=2, Hq=16, Hkv=2, d=128, dtype="bf16", split=128, N=1)
    inp = synth.make_inputs(synth.with_lens(base, (1000, 333)))
    r = Run(inp)
    sync = _skip_unsupported(lambda: r.run(kernel=kernel))
    allf = r.run(kernel=kernel, mode="unified", phi=0.0, lo=64.0, hi=64.0)   # every score < lo
    valid = sync["part_l"] > 0
    assert np.array_equal(allf["flags"].astype(bool), valid)
    assert allf["count"] == int(valid.sum())
    for key in ("out", "lse", "part_m", "part_l"):
        assert np.array_equal(allf[key], sync[key]), key
    assert np.array_equal(allf["part_o"][valid], sync["part_o"][valid])


@pytest.mark.parametrize("kernel", KERNELS)
def test_unified_max_no_flags_in_a_wide_range(kernel):
    base = synth.Workload("umax_none", B=2, Hq=16, Hkv=2, d=128, dtype="bf16", split=128, N=1)
    inp = synth.make_inputs(synth.with_lens(base, (1000, 333)))
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel, mode="unified", phi=-30.0, lo=-30.0, hi=30.0))
    assert res["count"] == 0 and not res["flags"].any()
    ft.check_exact(res, inp, what="unified, nothing flagged")
    valid = res["part_l"] > 0
    assert np.all(np.abs(res["part_m"][valid] - (-30.0)) < 1e-5)


@pytest.mark.parametrize("kernel", ["auto"] + KERNELS)
@pytest.mark.parametrize("dtype,d", [("f16", 128), ("f32", 128), ("f16", 64), ("f32", 64), ("bf16", 64)])
def test_unified_max_dtypes_and_head_dims(kernel, dtype, d):
    """Unified max beyond bf16 at d = 128: f16 and f32 caches (the VALU kernel;
    the MFMA kernel reports f32 caches and f16 q in this mode unsupported) and
    d = 64.  Flags within the oracle's must/may sets, the fallback count, out
    and lse on every row, and the partials of every split whose flag agrees."""
    import oracle
    base = synth.Workload("umaxdt", B=2, Hq=16, Hkv=4, d=d, dtype=dtype, split=256, N=1,
                          stress_frac=0.02, stress_scale=8.0)
    inp = synth.make_inputs(synth.with_lens(base, (3000, 700)))
    w = inp.w
    S = -(-w.N // w.split)
    phi, lo, hi = -12.0, -12.0, 12.0
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel, mode="unified", phi=phi, lo=lo, hi=hi))
    must, may = ft.flag_bounds(inp, w.split, S, phi, lo, hi)
    got = res["flags"].astype(bool)
    assert np.all(got[must]) and not np.any(got[~may])
    assert res["count"] == int(got.sum()) and 0 < got.sum() < got.size
    what = f"unified {kernel} {dtype} d={d}"
    ft.check_exact(res, inp, what=what)
    uo = oracle.unified_max(oracle.problem_of(inp), inp.q, inp.k, inp.v, w.split, S, phi, lo, hi,
                            seq_lens=inp.seq_lens)
    agree = (uo["flags"].astype(bool) == got) & (uo["part_l"] > 0)
    for key in ("part_m", "part_l", "part_o"):
        ft.assert_close(res[key][agree], uo[key][agree], dtype, f"{what} {key}")


# ----------------------------------------------------------------------------
# 8-bit (OCP E4M3) caches with per-tensor scales
# ----------------------------------------------------------------------------
def _fp8_workload(name, B, Hq, Hkv, d, qdt, lens, page=0, split=256, ks=1.0 / 64, vs=1.0 / 64, **kw):
    base = synth.Workload(name, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype="fp8", split=split, N=1, page_size=page,
                          qdtype=qdt, k_scale=ks, v_scale=vs, **kw)
    return synth.make_inputs(synth.with_lens(base, lens))


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("qdt", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8), (16, 2)])
def test_fp8_cache_shapes(kernel, qdt, d, Hq, Hkv):
    inp = _fp8_workload("fp8", 3, Hq, Hkv, d, qdt, (1000, 1, 385), split=128, ks=0.037, vs=1.9)
    res = Run(inp).run(kernel=kernel)
    what = f"fp8 {kernel} q={qdt} d={d} G={Hq // Hkv}"
    ft.check_exact(res, inp, what=what)
    ft.check_partials(res, inp, 128, what=what)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("page", [0, 16])
def test_fp8_cache_equals_the_bf16_cache_of_its_values_bitwise(kernel, page):
    """Power-of-two scales make the dequantised values exact bf16 numbers, and
    the widening is exact: both caches give the same scores, hence the same
    bits of m, l and lse.  The VALU kernel also gives the same O bits.  The
    MFMA kernel takes P x V of an 8-bit cache in f16 (P rounded to nearest,
    relative error <= 2^-11) where the 16-bit cache takes P as a bf16 pair
    (<= 2^-14), so its O rows differ by at most about 2^-11 max|v|."""
    inp8 = _fp8_workload("fp8eq", 2, 32, 8, 128, "bf16", (3000, 517), page=page)
    w16 = dataclasses.replace(inp8.w, dtype="bf16", qdtype=None, k_scale=1.0, v_scale=1.0)
    k16 = synth.f32_to_bf16_bits((synth.decode_f64(inp8.k, "fp8") * inp8.w.k_scale).astype(np.float32))
    v16 = synth.f32_to_bf16_bits((synth.decode_f64(inp8.v, "fp8") * inp8.w.v_scale).astype(np.float32))
    inp16 = synth.Inputs(w16, inp8.q, k16, v16, inp8.seq_lens, inp8.block_table)
    a = Run(inp8).run(kernel=kernel)
    b = Run(inp16).run(kernel=kernel)
    for key in ("lse", "part_m", "part_l"):
        assert np.array_equal(a[key], b[key]), key
    valid = a["part_l"] > 0
    if kernel == "valu":
        assert np.array_equal(a["out"], b["out"])
        assert np.array_equal(a["part_o"][valid], b["part_o"][valid])
    else:
        vmax = float(np.nanmax(np.abs(synth.decode_f64(inp8.v, "fp8") * inp8.w.v_scale)))   # poisoned tail: NaN codes
        tol = 2.0 ** -10 * vmax
        assert np.abs(a["part_o"][valid] - b["part_o"][valid]).max() <= tol
        # out is rounded to bf16 on top: at most one unit in the last place apart
        assert np.abs(a["out"].astype(np.float64) - b["out"]).max() <= tol + 2.0 ** -7 * vmax
    ft.check_exact(a, inp8, what=f"fp8 {kernel} page={page}")


def test_fp8_paged_batched_shape():
    inp = _fp8_workload("fp8paged", 6, 64, 8, 128, "bf16", (16384, 1024, 7000, 16, 4097, 2500), page=16)
    res = Run(inp).run()
    ft.check_exact(res, inp, what="fp8 paged")
    ft.check_partials(res, inp, 256, what="fp8 paged")


@pytest.mark.parametrize("qdt", ["bf16", "f16"])
def test_fp8_unified_max_flags_and_fallback(qdt):
    inp = _fp8_workload("fp8umax", 2, 32, 4, 128, qdt, (4096, 1500), stress_frac=0.02, stress_scale=8.0)
    w = inp.w
    S = -(-w.N // w.split)
    phi, lo, hi = -12.0, -12.0, 12.0
    res = Run(inp).run(mode="unified", phi=phi, lo=lo, hi=hi)
    must, may = ft.flag_bounds(inp, w.split, S, phi, lo, hi)
    got = res["flags"].astype(bool)
    assert np.all(got[must]) and not np.any(got[~may])
    assert res["count"] == int(got.sum()) and 0 < got.sum() < got.size
    ft.check_exact(res, inp, what=f"fp8 unified q={qdt}")


def test_fp8_long_context_gqa_full():
    w = synth.WORKLOADS["long_gqa_32k_fp8"]
    say("[long_gqa_32k_fp8] generating")
    inp = synth.make_inputs(w)
    res = Run(inp).run()
    e1, e2 = ft.check_exact(res, inp, what="long_gqa_32k_fp8")
    ft.check_partials(res, inp, w.split, what="long_gqa_32k_fp8")
    say(f"[long_gqa_32k_fp8] max|out err|={e1:.3e} max|lse err|={e2:.3e}")


# ----------------------------------------------------------------------------
# several causal query tokens per request (draft verification / a chunk of new
# tokens already in the cache); q_len * G rows share one KV head
# ----------------------------------------------------------------------------
MQ_CASES = [  # (kernel, dtype, Hq, Hkv, q_len, d)
    ("mfma", "bf16", 32, 8, 4, 128), ("mfma", "bf16", 8, 8, 16, 128), ("mfma", "f16", 16, 8, 8, 128),
    ("mfma", "bf16", 24, 8, 5, 128), ("mfma", "fp8", 32, 8, 4, 128), ("mfma", "bf16", 16, 4, 3, 64),
    ("valu", "f32", 16, 8, 3, 128), ("valu", "bf16", 32, 8, 4, 128), ("valu", "fp8", 8, 8, 2, 128),
    ("valu", "f16", 8, 2, 4, 64),
    # more than 16 rows: two 16-row tiles per KV head (MFMA kernel only)
    ("mfma", "bf16", 64, 8, 4, 128), ("mfma", "f16", 24, 8, 7, 64), ("mfma", "fp8", 32, 4, 3, 128),
    ("mfma", "bf16", 8, 8, 32, 128),
]


@pytest.mark.parametrize("page", [0, 16])
@pytest.mark.parametrize("kernel,dtype,Hq,Hkv,q_len,d", MQ_CASES)
def test_multi_query_causal(kernel, dtype, Hq, Hkv, q_len, d, page):
    extra = dict(k_scale=1.0 / 64, v_scale=1.0 / 64) if dtype == "fp8" else {}
    base = synth.Workload("mq", B=1, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, split=128, N=1, page_size=page,
                          q_len=q_len, **extra)
    # lengths cover a split boundary inside the query window and a request
    # shorter than its query tokens
    inp = synth.make_inputs(synth.with_lens(base, (1000, 129, 130, 3, 2 * q_len)))
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel))
    what = f"q_len={q_len} {kernel} {dtype} d={d} G={Hq // Hkv} page={page}"
    ft.check_exact(res, inp, what=what)
    ft.check_partials(res, inp, 128, what=what)
    # query token 0 of the request of length 3 < q_len sees nothing when q_len > 3
    if q_len > 3:
        r0 = (3 * q_len + 0) * Hq
        assert np.all(res["out"][r0:r0 + Hq] == 0.0) and np.all(res["lse"][r0:r0 + Hq] == -np.inf)


# ----------------------------------------------------------------------------
# query tiles: more query rows per KV head than a workgroup holds (32 MFMA,
# 16 VALU), e.g. a prefill chunk or a whole prompt; the rows go in tiles of
# whole query tokens, each reading only the cache tokens its rows can see
# ----------------------------------------------------------------------------
QT_CASES = [  # (kernel, dtype, Hq, Hkv, q_len, d): tiles of the kernel's rows
    ("mfma", "bf16", 32, 8, 20, 128),     # G=4, 80 rows: tiles of 7, 7, 6 tokens
    ("mfma", "f16", 8, 8, 100, 128),      # G=1, 100 rows: 4 tiles of 25
    ("mfma", "fp8", 64, 8, 9, 128),       # G=8, 72 rows: 3 tiles of 3
    ("mfma", "bf16", 16, 4, 70, 64),      # G=4, 280 rows: 9 tiles (8 tokens, the last 6)
    ("valu", "f32", 16, 8, 20, 128),      # G=2, 40 rows: tiles of 7, 7, 6
    ("valu", "bf16", 8, 8, 40, 64),       # G=1: tiles of 14, 14, 12
    ("valu", "fp8", 32, 8, 6, 128),       # G=4: 2 tiles of 3
    ("auto", "f32", 64, 8, 4, 128),       # G=8, 32 rows: 2 VALU tiles of 2 tokens
    # four or more tiles: workgroups of four tiles sharing each K/V block
    ("mfma", "fp8", 32, 8, 40, 128),      # G=4: 5 tiles of 8 (a second group with one tile)
    ("mfma", "bf16", 64, 8, 33, 128),     # G=8: 9 tiles (4 tokens, the last 1)
    ("mfma", "f16", 16, 16, 150, 64),     # G=1: 5 tiles of 30
]


def _tile_inputs(dtype, Hq, Hkv, q_len, d, page=0, split=128, **kw):
    extra = dict(k_scale=1.0 / 64, v_scale=1.0 / 64) if dtype == "fp8" else {}
    extra.update(kw)
    base = synth.Workload("qt", B=1, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, split=split, N=1, page_size=page,
                          q_len=q_len, **extra)
    # a request as long as its query tokens (a whole prompt), shorter ones (the
    # early tiles see nothing), and longer ones across split boundaries
    return synth.make_inputs(synth.with_lens(base, (1000, 3, q_len, 2 * q_len + 129, 257)))


@pytest.mark.parametrize("page", [0, 16])
@pytest.mark.parametrize("kernel,dtype,Hq,Hkv,q_len,d", QT_CASES)
def test_query_tiles(kernel, dtype, Hq, Hkv, q_len, d, page):
    inp = _tile_inputs(dtype, Hq, Hkv, q_len, d, page)
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel, merge="separate"))
    what = f"tiles q_len={q_len} {kernel} {dtype} d={d} G={Hq // Hkv} page={page}"
    ft.check_exact(res, inp, what=what)
    ft.check_partials(res, inp, 128, what=what)
    # the request of 3 tokens: its query tokens before the last 3 see nothing
    r0 = (1 * q_len) * Hq
    n_blind = (q_len - 3) * Hq
    assert np.all(res["out"][r0:r0 + n_blind] == 0.0) and np.all(res["lse"][r0:r0 + n_blind] == -np.inf)


@pytest.mark.parametrize("page", [32, 64])
@pytest.mark.parametrize("kernel,dtype,Hq,Hkv,q_len,d", QT_CASES[8:11])
def test_query_tile_groups_large_pages(kernel, dtype, Hq, Hkv, q_len, d, page):
    """Tile groups sharing K/V blocks over pages of 32 and 64 tokens (each
    16-token block inside one page, several blocks per page): split partials,
    and with one split per row (split 1024) the result written directly."""
    inp = _tile_inputs(dtype, Hq, Hkv, q_len, d, page)
    what = f"tile groups q_len={q_len} {kernel} {dtype} d={d} page={page}"
    res = Run(inp).run(kernel=kernel, merge="separate")
    ft.check_exact(res, inp, what=what)
    ft.check_partials(res, inp, 128, what=what)
    inp = _tile_inputs(dtype, Hq, Hkv, q_len, d, page, split=1024)
    res = Run(inp).run(kernel=kernel, full=True)
    ft.check_exact(res, inp, what=what + " direct")


@pytest.mark.parametrize("kernel,dtype,Hq,Hkv,q_len,d", [QT_CASES[0], QT_CASES[3], QT_CASES[4], QT_CASES[5]])
def test_query_tiles_single_launch(kernel, dtype, Hq, Hkv, q_len, d):
    """The single-launch merge with one counter per (request, tile, KV head)."""
    inp = _tile_inputs(dtype, Hq, Hkv, q_len, d)
    for _ in range(2):                                  # counters left zero for the next call
        res = Run(inp).run(kernel=kernel, full=True, merge="fused")
        ft.check_exact(res, inp, what=f"tiles fused q_len={q_len} {kernel} {dtype}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("fallback", ["split", "row"])
def test_query_tiles_unified_max(kernel, fallback):
    inp = _tile_inputs("bf16", 32, 8, 12, 128, stress_frac=0.02, stress_scale=8.0)
    w = inp.w
    S = -(-w.N // w.split)
    phi, lo, hi = -12.0, -12.0, 12.0
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel, mode="unified", phi=phi, lo=lo, hi=hi,
                                                 fallback=fallback))
    must, may = ft.flag_bounds(inp, w.split, S, phi, lo, hi)
    got = res["flags"].astype(bool)
    assert np.all(got[must]) and not np.any(got[~may])
    assert 0 < got.sum() < got.size
    ft.check_exact(res, inp, what=f"tiles unified {kernel} {fallback}")


def test_query_tiles_match_untiled_rows_bitwise():
    """A tile's rows are computed as they are without tiles: the VALU kernel
    (16 rows per workgroup) on 32 rows in two tiles gives the bits of the
    same rows run as two calls of 16 rows each (the last q_len / 2 tokens,
    and the first q_len / 2 at a request length shortened by q_len / 2)."""
    w = synth.Workload("qtb", B=1, Hq=8, Hkv=2, d=128, dtype="bf16", split=128, N=1, q_len=8)
    inp = synth.make_inputs(synth.with_lens(w, (900, 300)))
    res = Run(inp).run(kernel="valu")
    w = inp.w
    half = w.q_len // 2
    for part, (i0, cut) in enumerate(((0, half), (half, 0))):
        lens = inp.seq_lens - cut
        w1 = dataclasses.replace(w, q_len=half, fixed_lens=tuple(int(x) for x in lens), name="qtb1")
        inp1 = synth.Inputs(w1, np.ascontiguousarray(inp.q[:, i0:i0 + half]), inp.k, inp.v,
                            lens.astype(np.int32))
        r1 = Run(inp1).run(kernel="valu")
        for b in range(w.B):
            r = slice((b * w.q_len + i0) * w.Hq, (b * w.q_len + i0 + half) * w.Hq)
            r_1 = slice(b * half * w.Hq, (b + 1) * half * w.Hq)
            assert np.array_equal(res["out"][r], r1["out"][r_1]), (part, b)
            assert np.array_equal(res["lse"][r], r1["lse"][r_1]), (part, b)


# ----------------------------------------------------------------------------
# one split per row (max_splits == 1): under AUTO the partial kernel writes
# out and lse itself, with no partials and no merge
# ----------------------------------------------------------------------------
DIRECT_CASES = [  # (kernel, dtype, Hq, Hkv, q_len, d)
    ("mfma", "bf16", 32, 8, 1, 128), ("mfma", "f16", 8, 8, 1, 64), ("mfma", "fp8", 32, 8, 1, 128),
    ("mfma", "bf16", 32, 8, 20, 128), ("valu", "f32", 16, 8, 1, 128), ("valu", "bf16", 8, 8, 40, 64),
    ("mfma", "bf16", 32, 8, 40, 128), ("mfma", "fp8", 16, 16, 130, 64),   # shared-K/V tile groups
]


@pytest.mark.parametrize("page", [0, 16])
@pytest.mark.parametrize("kernel,dtype,Hq,Hkv,q_len,d", DIRECT_CASES)
def test_direct_single_split(kernel, dtype, Hq, Hkv, q_len, d, page):
    extra = dict(k_scale=1.0 / 64, v_scale=1.0 / 64) if dtype == "fp8" else {}
    base = synth.Workload("direct", B=1, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, split=1024, N=1, page_size=page,
                          q_len=q_len, **extra)
    # an empty request, one shorter than its query tokens, one at the split's size
    inp = synth.make_inputs(synth.with_lens(base, (700, 0, 3, 1024, 129)))
    run = Run(inp)
    res = _skip_unsupported(lambda: run.run(kernel=kernel, full=True))
    assert res["desc"].max_splits == 1
    what = f"direct {kernel} {dtype} q_len={q_len} d={d} page={page}"
    ft.check_exact(res, inp, what=what)
    r0 = q_len * Hq                                  # the empty request's rows
    assert np.all(res["out"][r0:2 * r0] == 0.0) and np.all(res["lse"][r0:2 * r0] == -np.inf)
    sep = run.run(kernel=kernel, full=True, merge="separate")
    # (the direct launch takes one-wave workgroups, the separate one may take
    # two, which round the split's sums in another order)
    ft.assert_close(res["out"], sep["out"], dtype, f"{what} vs separate")
    ft.assert_close(res["lse"], sep["lse"], dtype, f"{what} lse vs separate")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_direct_tiles_with_score_spikes(dtype):
    """One split per row, query tiles sharing K/V, direct output: the running
    reference maximum moves only on jumps beyond 2^8 in the weights there.
    Keys scaled x8 on 5% of the rows make the scores jump by tens of units
    anywhere in the sequence; every row against the oracle."""
    base = synth.Workload("spikes", B=1, Hq=32, Hkv=8, d=128, dtype=dtype, split=4096, N=1, q_len=64,
                          stress_frac=0.05, stress_scale=8.0)
    inp = synth.make_inputs(synth.with_lens(base, (3000, 64, 900)))
    res = Run(inp).run(full=True)
    assert res["desc"].max_splits == 1
    ft.check_exact(res, inp, what=f"direct spikes {dtype}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("fallback", ["split", "row"])
def test_single_split_unified_max(kernel, fallback):
    """One split per row under unified max: AUTO keeps the partials and the
    merge there (the direct output is the synchronized softmax's)."""
    base = synth.Workload("directu", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", split=2048, N=1, q_len=2,
                          stress_frac=0.02, stress_scale=8.0)
    inp = synth.make_inputs(synth.with_lens(base, (2000, 700, 1)))
    phi, lo, hi = -12.0, -12.0, 12.0
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel, full=True, mode="unified", phi=phi, lo=lo, hi=hi,
                                                 fallback=fallback))
    must, may = ft.flag_bounds(inp, 2048, 1, phi, lo, hi)
    got = res["flags"].astype(bool)
    assert np.all(got[must]) and not np.any(got[~may]) and got.any()
    ft.check_exact(res, inp, what=f"single split unified {kernel} {fallback}")


@pytest.mark.parametrize("split,merge", [(65536, "auto"), (8192, "separate"), (8192, "fused")])
def test_max_query_tokens(split, merge):
    """The largest q_len (FD_MAX_Q_LEN = 65,536): a whole prompt of that
    length as queries (2 query heads on 1 KV head, d=64), 2,048 query tiles
    per KV head: one split (direct output from the groups sharing K/V),
    eight splits with the combine, and eight with the single-launch merge.
    Rows sampled across the prompt, the first and last tokens included,
    against the oracle one by one."""
    import decode_attention_attn_amd as fd
    n = fd.MAX_Q_LEN
    w = synth.Workload("qmax", B=1, Hq=2, Hkv=1, d=64, dtype="bf16", split=split, N=n, q_len=n)
    inp = synth.make_inputs(w)
    res = Run(inp).run(full=True, merge=merge)
    assert res["desc"].max_splits == n // split
    R = n * w.Hq
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(R - 8, R), ft.sample_rows(w, 240, seed=5)]))
    ft.check_exact(res, inp, rows=rows.astype(np.int32), what=f"q_len={n} split={split} {merge}")


def test_paged_batch_short_full():
    """256 short requests (1..1000 tokens, paged): one split per row, the
    paged entry point's AUTO writes the result from the partial kernel;
    every row against the oracle, and against the separate merge."""
    w = synth.WORKLOADS["paged_batch_short"]
    inp = synth.make_inputs(w)
    run = Run(inp)
    res = run.run()
    assert res["desc"].max_splits == 1
    e1, e2 = ft.check_exact(res, inp, what=w.name)
    sep = run.run(merge="separate")
    ft.check_exact(sep, inp, what=f"{w.name} separate")
    ft.check_partials(sep, inp, w.split, what=w.name)
    say(f"[{w.name}] max|out err|={e1:.3e} max|lse err|={e2:.3e}")


def test_prefill_gqa_4k_full():
    """A whole 4k prompt as queries (32 heads on 8 KV heads, one split): every
    row against the oracle, through the AUTO entry point (direct output) and
    the partial + combine kernels."""
    w = synth.WORKLOADS["prefill_gqa_4k"]
    say(f"[{w.name}] generating")
    inp = synth.make_inputs(w)
    run = Run(inp)
    res = run.run(full=True)
    e1, e2 = ft.check_exact(res, inp, what=w.name)
    say(f"[{w.name}] direct max|out err|={e1:.3e} max|lse err|={e2:.3e}")
    res = run.run()
    ft.check_exact(res, inp, what=f"{w.name} partial + combine")
    ft.check_partials(res, inp, w.split, what=w.name)


@pytest.mark.parametrize("q_len,Hq", [(4, 16), (4, 64)])
@pytest.mark.parametrize("kernel", KERNELS)
def test_multi_query_unified_max(kernel, q_len, Hq):
    Hkv = 4 if Hq == 16 else 8
    if kernel == "valu" and q_len * (Hq // Hkv) > 16:
        pytest.skip("the VALU kernel holds up to 16 rows")
    base = synth.Workload("mqu", B=1, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", split=256, N=1,
                          q_len=q_len, stress_frac=0.02, stress_scale=8.0)
    inp = synth.make_inputs(synth.with_lens(base, (3000, 700)))
    w = inp.w
    S = -(-w.N // w.split)
    phi, lo, hi = -12.0, -12.0, 12.0
    res = _skip_unsupported(lambda: Run(inp).run(kernel=kernel, mode="unified", phi=phi, lo=lo, hi=hi))
    must, may = ft.flag_bounds(inp, w.split, S, phi, lo, hi)
    got = res["flags"].astype(bool)
    assert np.all(got[must]) and not np.any(got[~may])
    assert res["count"] == int(got.sum()) and 0 < got.sum() < got.size
    ft.check_exact(res, inp, what=f"q_len={q_len} Hq={Hq} unified {kernel}")


def test_multi_query_rows_match_single_query_runs_bitwise():
    """Each query row equals a one-token decode of the same q row at its causal
    length, run through the library: same split boundaries and, with q_len * G
    and G both at most 4, the same two-wave launch shape (rows of a matrix
    tile are computed independently), so the same bits."""
    base = synth.Workload("mqs", B=1, Hq=16, Hkv=8, d=128, dtype="bf16", split=256, N=1, q_len=2)
    inp = synth.make_inputs(synth.with_lens(base, (2000, 513)))
    res = Run(inp).run(kernel="mfma")
    w = inp.w
    for b in range(w.B):
        for i in range(w.q_len):
            n = int(inp.seq_lens[b]) - w.q_len + i + 1
            w1 = dataclasses.replace(w, B=1, q_len=1, N=w.N, fixed_lens=(n,), name="mqs1")
            inp1 = synth.Inputs(w1, inp.q[b, i][None].copy(), inp.k[b:b + 1].copy(), inp.v[b:b + 1].copy(),
                                np.array([n], np.int32))
            r1 = Run(inp1).run(kernel="mfma")
            r = slice((b * w.q_len + i) * w.Hq, (b * w.q_len + i + 1) * w.Hq)
            assert np.array_equal(res["lse"][r], r1["lse"]), (b, i)
            assert np.array_equal(res["out"][r], r1["out"]), (b, i)


@pytest.mark.parametrize("name", ["long_gqa_32k_verify4", "long_gqa_32k_verify8"])
def test_verify_tokens_long_context_gqa_full(name):
    w = synth.WORKLOADS[name]
    say(f"[{name}] generating")
    inp = synth.make_inputs(w)
    res = Run(inp).run()
    e1, e2 = ft.check_exact(res, inp, what=name)
    ft.check_partials(res, inp, w.split, what=name)
    say(f"[{name}] max|out err|={e1:.3e} max|lse err|={e2:.3e}")


# ----------------------------------------------------------------------------
# the split the heuristic picks is a valid launch for every kernel
# ----------------------------------------------------------------------------
HEURISTIC_CASES = [  # (B, Hq, Hkv, lens, page)
    ((1, 32, 8, (32768,), 0)), ((1, 8, 8, (700,), 0)), ((4, 32, 32, (4096, 100, 3000, 1), 0)),
    ((2, 64, 8, (9000, 2049), 16)), ((3, 16, 16, (77, 300, 129), 16)),
    # a batch that fills the GPU several times over: one split per row (the paged
    # entry point then writes the result from the partial kernel, no merge)
    ((256, 32, 8, tuple(int(x) for x in np.random.default_rng(17).integers(1, 1001, 256)), 16)),
]


@pytest.mark.parametrize("B,Hq,Hkv,lens,page", HEURISTIC_CASES)
def test_heuristic_split_runs_and_matches_the_oracle(B, Hq, Hkv, lens, page):
    import decode_attention_attn_amd as fd
    split, S = fd.fd_split_heuristic(B, Hq, Hkv, max(lens), page, 256)
    base = synth.Workload("heur", B=B, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", split=split, N=1, page_size=page)
    inp = synth.make_inputs(synth.with_lens(base, lens))
    res = Run(inp).run()
    say(f"[heuristic] split={split} S={S} (cache S_max {res['part_m'].shape[1]})")
    ft.check_exact(res, inp, what=f"heuristic split {split}")
    if res["part_m"].shape[1] > 1 or not page:   # one split, paged (AUTO): no partials are written
        ft.check_partials(res, inp, split, what=f"heuristic split {split}")


# ----------------------------------------------------------------------------
# 8-bit caches with one scale per KV head
# ----------------------------------------------------------------------------
HEAD_KS = (0.011, 0.037, 0.0213, 0.05, 0.0077, 0.029, 0.017, 0.043)
HEAD_VS = (1.9, 0.7, 1.31, 0.43, 2.2, 1.05, 0.61, 1.7)


@pytest.mark.parametrize("page", [0, 16])
@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("Hq,Hkv,d,qdt", [(32, 8, 128, "bf16"), (16, 4, 64, "f16"), (8, 8, 128, "bf16")])
def test_fp8_per_head_scales(kernel, Hq, Hkv, d, qdt, page):
    inp = _fp8_workload("fp8heads", 3, Hq, Hkv, d, qdt, (1000, 1, 385), page=page, split=128,
                        k_scales=HEAD_KS[:Hkv], v_scales=HEAD_VS[:Hkv])
    res = Run(inp).run(kernel=kernel)
    what = f"fp8 per-head {kernel} q={qdt} d={d} G={Hq // Hkv} page={page}"
    ft.check_exact(res, inp, what=what)
    ft.check_partials(res, inp, 128, what=what)


@pytest.mark.parametrize("split,page", [(128, 0), (128, 16), (2048, 0), (2048, 16)])
def test_fp8_per_head_scales_query_tiles(split, page):
    """Per-head 8-bit scales with 40 query tokens per request: query tiles in
    groups sharing K/V, writing partials (split 128) or the result directly
    (split 2048, one split per row)."""
    inp = _fp8_workload("fp8tiles", 3, 32, 8, 128, "bf16", (1000, 40, 385), page=page, split=split,
                        k_scales=HEAD_KS, v_scales=HEAD_VS, q_len=40)
    res = Run(inp).run(full=True)
    what = f"fp8 per-head tiles split={split} page={page}"
    ft.check_exact(res, inp, what=what)


def test_fp8_per_head_scales_equal_to_the_tensor_scale_are_bitwise_the_same():
    """Per-head scales that all equal the tensor scale give the same bits as
    the tensor scale (power-of-two scales: the products are exact either way)."""
    a = _fp8_workload("fp8h1", 2, 32, 8, 128, "bf16", (3000, 517))
    b = _fp8_workload("fp8h2", 2, 32, 8, 128, "bf16", (3000, 517), k_scales=(1.0 / 64,) * 8,
                      v_scales=(1.0 / 64,) * 8)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    ra, rb = Run(a).run(), Run(b).run()
    for key in ("out", "lse", "part_m", "part_l"):
        assert np.array_equal(ra[key], rb[key]), key


def test_fp8_per_head_scales_full_size():
    w = synth.WORKLOADS["long_gqa_32k_fp8_head_scales"]
    say("[long_gqa_32k_fp8_head_scales] generating")
    inp = synth.make_inputs(w)
    res = Run(inp).run()
    e1, e2 = ft.check_exact(res, inp, what="fp8 per-head scales, 32k GQA")
    ft.check_partials(res, inp, w.split, what="fp8 per-head scales, 32k GQA")
    say(f"[long_gqa_32k_fp8_head_scales] max|out err|={e1:.3e} max|lse err|={e2:.3e}")
