"""Seeded random problems through the C ABI against the fp64 oracle.

Each case draws one problem from a fixed seed: cache dtype, head dimension,
KV heads and group size, batch, query tokens per request, contiguous or
paged cache (pages of 16 or 32 tokens), split size, request lengths from
empty to the cache capacity, kernel choice, softmax mode (the unified
maximum with and without out-of-range scores) and merge mode.  Every query
row's out and lse are compared with the oracle at the bar of fdtest.py, and
the split partials too where a separate merge leaves them in the caller's
buffers.  A second draw covers the whole-row fallback, per-KV-head 8-bit
scales and query blocks long enough for several query tiles.  Combinations
the library reports unsupported are skipped.
"""
import numpy as np
import pytest

import fdtest as ft
from fdtest import Run, say
import synth

pytestmark = pytest.mark.gpu

N_CASES = 160


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = ft.torch()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_attn_amd as fd
    fd.lib()


def _draw(seed):
    rng = np.random.default_rng(20260 + seed)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    dtype = pick(["f32", "f16", "bf16", "bf16", "fp8"])
    d = pick([64, 128])
    Hkv = pick([1, 2, 4, 8])
    G = pick([1, 2, 4, 8])
    B = int(rng.integers(1, 7))
    q_len = pick([1, 1, 1, 2, 3, 5, 9, 17])
    page = pick([0, 0, 16, 32])
    split = pick([32, 64, 128, 256, 512] if page else [16, 48, 64, 128, 256, 512])
    N = int(rng.integers(1, 4097))
    lens = [int(x) for x in rng.integers(0, N + 1, size=B)]
    if B > 1 and rng.integers(4) == 0:
        lens[int(rng.integers(B))] = 0                 # an empty request among others
    lens = tuple(lens)
    mode = pick(["sync", "sync", "unified"])
    extra = {}
    if dtype == "fp8":
        extra = dict(k_scale=1.0 / 64, v_scale=1.0 / 64, qdtype=pick(["bf16", "f16"]))
    # the MFMA kernel takes no fp32 cache, nor f16 operands under the unified maximum
    f16_ops = dtype == "f16" or extra.get("qdtype") == "f16"
    kernel = pick(["auto", "valu"] if dtype == "f32" or (f16_ops and mode == "unified") else ["auto", "mfma", "valu"])
    merge = pick(["auto", "separate", "fused"])
    stress = mode == "unified" and bool(rng.integers(2))
    if stress:
        extra.update(stress_frac=0.02, stress_scale=8.0)
    w = synth.Workload(f"rand{seed}", B=B, Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, split=split, N=N,
                       page_size=page, q_len=q_len, **extra)
    return synth.with_lens(w, lens), kernel, mode, merge


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_problem(seed):
    import decode_attention_attn_amd as fd
    w, kernel, mode, merge = _draw(seed)
    what = (f"seed={seed} {w.dtype} d={w.d} Hq={w.Hq} Hkv={w.Hkv} B={w.B} q_len={w.q_len} "
            f"page={w.page_size} split={w.split} lens={w.fixed_lens} {kernel} {mode} {merge}")
    say(what)
    inp = synth.make_inputs(w)
    kw = dict(kernel=kernel, mode=mode, merge=merge)
    if mode == "unified":
        kw.update(phi=-10.0, lo=-10.0, hi=10.0)
    separate = not w.page_size and merge == "separate"
    try:
        res = Run(inp).run(full=not separate, **kw)
    except fd.FdError as e:
        if e.status == fd.FD_ERR_UNSUPPORTED:
            pytest.skip(f"unsupported: {what}")
        raise
    ft.check_exact(res, inp, what=what)
    if separate and mode == "sync":
        ft.check_partials(res, inp, w.split, what=what)


N_EXTRA = 64


def _draw_extra(seed):
    """Axes the first draw leaves out: the whole-row fallback (its second
    launch needs the separate merge), per-KV-head 8-bit scales, and longer
    query blocks (several query tiles, the tile groups that share K and V)."""
    rng = np.random.default_rng(90210 + seed)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    kind = pick(["row_fallback", "head_scales", "long_query"])
    d = pick([64, 128])
    Hkv = pick([1, 2, 4, 8])
    G = pick([1, 2, 4, 8])
    B = int(rng.integers(1, 5))
    page = pick([0, 16])
    extra, kernel, mode, merge, fallback = {}, pick(["auto", "mfma", "valu"]), "sync", "auto", "split"
    if kind == "row_fallback":
        dtype, q_len, split = pick(["bf16", "f16", "f32"]), pick([1, 2, 5]), pick([64, 128, 256])
        mode, merge, fallback = "unified", "separate", "row"
        extra.update(stress_frac=0.02, stress_scale=8.0)
        if dtype != "bf16":
            kernel = pick(["auto", "valu"])
    elif kind == "head_scales":
        dtype, q_len, split = "fp8", pick([1, 1, 3, 9]), pick([64, 128, 256])
        scales = rng.uniform(0.004, 0.05, size=(2, Hkv))
        extra.update(k_scales=tuple(float(x) for x in scales[0]), v_scales=tuple(float(x) for x in scales[1]),
                     qdtype=pick(["bf16", "f16"]))
        merge = pick(["auto", "separate", "fused"])
    else:
        dtype, q_len, split = pick(["bf16", "f16", "fp8"]), pick([24, 40, 65]), pick([128, 512, 4096])
        if dtype == "fp8":
            extra.update(k_scale=1.0 / 64, v_scale=1.0 / 64)
        merge = pick(["auto", "separate"])
    lens = tuple(int(x) for x in rng.integers(0, 3001, size=B))
    w = synth.Workload(f"randx{seed}", B=B, Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, split=split, N=1,
                       page_size=page, q_len=q_len, **extra)
    return synth.with_lens(w, lens), kernel, mode, merge, fallback


@pytest.mark.parametrize("seed", range(N_EXTRA))
def test_random_problem_more_axes(seed):
    import decode_attention_attn_amd as fd
    w, kernel, mode, merge, fallback = _draw_extra(seed)
    what = (f"seed={seed} {w.dtype} d={w.d} Hq={w.Hq} Hkv={w.Hkv} B={w.B} q_len={w.q_len} "
            f"page={w.page_size} split={w.split} lens={w.fixed_lens} {kernel} {mode} {merge} {fallback}")
    say(what)
    inp = synth.make_inputs(w)
    kw = dict(kernel=kernel, mode=mode, merge=merge, fallback=fallback)
    if mode == "unified":
        kw.update(phi=-10.0, lo=-10.0, hi=10.0)
    separate = not w.page_size and merge == "separate"
    try:
        res = Run(inp).run(full=not separate, **kw)
    except fd.FdError as e:
        if e.status == fd.FD_ERR_UNSUPPORTED:
            pytest.skip(f"unsupported: {what}")
        raise
    ft.check_exact(res, inp, what=what)
    if separate and mode == "sync":
        ft.check_partials(res, inp, w.split, what=what)
