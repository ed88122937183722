"""The merge of split partials on its own: fd_decode_attn_combine on hand-made
partials, against the oracle's fp64 merge.

The partial kernel never writes the O row of a split without tokens, so the
rule that such splits are skipped (Flash-Decoding page, "The Rescaling and
Online Softmax Reduction Algorithm"; handbook page "FlashAttention and
inference kernels", exercise 2) is only observable with partials that hold
garbage there.  Here every skipped O row is NaN, skipped m and l values are
garbage, and the split maxima spread over +-80, so a combine that reads a
skipped row, weighs it, or lets exp overflow returns NaN or a wrong value.
Both instantiations run: one request (O loads issued before the length is
known) and a batch with lengths (O loads only for the request's splits).
"""
import numpy as np
import pytest

import fdtest as ft
from fdtest import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = ft.torch()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_attn_amd as fd
    fd.lib()


def _partials(B, Hq, S, d, seed):
    """Random partials [B, Hq, S, d] / [B, Hq, S] with the special rows of the
    module docstring: row 0 of each request has an empty split in mid-row,
    row 1 is all empty, row 2 spreads its maxima over [-80, 80], row 3 has
    one non-empty split."""
    rng = np.random.default_rng(seed)
    po = rng.standard_normal((B, Hq, S, d)).astype(np.float32)
    pm = rng.uniform(-5.0, 5.0, (B, Hq, S)).astype(np.float32)
    pl = rng.uniform(1.0, 256.0, (B, Hq, S)).astype(np.float32)
    for b in range(B):
        mid = S // 2
        pm[b, 0, mid], pl[b, 0, mid], po[b, 0, mid] = -np.inf, 0.0, np.nan
        pm[b, 1, :], pl[b, 1, :], po[b, 1, :] = -np.inf, 0.0, np.nan
        pm[b, 2, :] = rng.uniform(-80.0, 80.0, S).astype(np.float32)
        pm[b, 2, 0], pm[b, 2, S - 1] = -80.0, 80.0
        keep = S - 1
        pm[b, 3, :keep], pl[b, 3, :keep], po[b, 3, :keep] = -np.inf, 0.0, np.nan
    return po, pm, pl


def _run_combine(po, pm, pl, split, lens):
    import decode_attention_attn_amd as fd
    t = ft.torch()
    B, Hq, S, d = po.shape
    desc = fd.make_desc(B, Hq, Hq, d, "f32", "f32", split_size=split, max_splits=S)
    dpo, dpm, dpl = (t.from_numpy(np.ascontiguousarray(a)).cuda() for a in (po, pm, pl))
    out = t.full((B, Hq, d), 7.0, dtype=t.float32, device="cuda")
    lse = t.full((B, Hq), 7.0, dtype=t.float32, device="cuda")
    dl = None if lens is None else t.from_numpy(np.asarray(lens, np.int32)).cuda()
    fd.fd_decode_attn_combine(desc, dpo, dpm, dpl, dl, out, lse)
    t.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _expect(po, pm, pl, split, lens):
    """The oracle's merge over the splits each request has (all without lengths)."""
    import oracle
    B, Hq, S, d = po.shape
    out = np.empty((B, Hq, d))
    lse = np.empty((B, Hq))
    for b in range(B):
        n = S if lens is None else min(S, -(-max(int(lens[b]), 0) // split))
        if n == 0:
            out[b], lse[b] = 0.0, -np.inf
            continue
        o, l_ = oracle.merge(po[b, :, :n].astype(np.float64), pm[b, :, :n].astype(np.float64),
                             pl[b, :, :n].astype(np.float64))
        out[b], lse[b] = o, l_
    return out, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", [1, 7, 64, 300])
def test_combine_one_request_hand_made_partials(S, d):
    po, pm, pl = _partials(1, 8, S, d, seed=S + d)
    if S == 1:      # rows 0 and 3 would otherwise be all empty too
        pm[0, 0, 0], pl[0, 0, 0], po[0, 0, 0] = 1.5, 3.0, 0.25
        pm[0, 3, 0], pl[0, 3, 0], po[0, 3, 0] = -2.0, 1.0, -0.5
    for lens in (None, [S * 64]):
        out, lse = _run_combine(po, pm, pl, 64, lens)
        ref, lref = _expect(po, pm, pl, 64, lens)
        say(f"[combine] S={S} d={d} lens={lens}")
        assert not np.isnan(out).any() and not np.isnan(lse).any()
        ft.assert_close(out, ref, "f32", "combine out")
        ft.assert_close(lse, lref, "f32", "combine lse")
        assert np.all(out[0, 1] == 0.0) and lse[0, 1] == -np.inf


def test_combine_batch_with_lengths_reads_only_each_requests_splits():
    """Splits past a request's last one hold NaN O rows and garbage m and l
    (m = 1000, l = 5): the combine must not read them.  One request is
    empty (out 0, lse -inf), one has a partial last split."""
    B, Hq, S, d, split = 4, 16, 40, 128, 32
    po, pm, pl = _partials(B, Hq, S, d, seed=3)
    lens = [S * split, 0, 10 * split + 5, 1]
    for b, n in enumerate(lens):
        used = -(-n // split)
        po[b, :, used:] = np.nan
        pm[b, :, used:] = 1000.0
        pl[b, :, used:] = 5.0
        if used == 1:   # the one split a length-1 request has: keep row 0 and row 3 non-empty
            pm[b, 0, 0], pl[b, 0, 0], po[b, 0, 0] = 0.5, 1.0, 1.0
            pm[b, 3, 0], pl[b, 3, 0], po[b, 3, 0] = 0.5, 1.0, 1.0
    out, lse = _run_combine(po, pm, pl, split, lens)
    ref, lref = _expect(po, pm, pl, split, lens)
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    ft.assert_close(out, ref, "f32", "combine out")
    ft.assert_close(lse, lref, "f32", "combine lse")
    assert np.all(out[1] == 0.0) and np.all(lse[1] == -np.inf)


# ----------------------------------------------------------------------------
# the single-launch merge (FD_MERGE_FUSED): the last workgroup of each
# (request, KV head) merges its partials inside the partial kernel
# ----------------------------------------------------------------------------

import synth
from fdtest import Run

FUSED_CASES = [  # (Hq, Hkv, lens, page, split)
    (32, 8, (4096, 1500, 17, 0, 257), 0, 256),        # ragged, an empty request, S = 16: four splits a group
    (32, 8, (4096, 1500, 17, 0, 257), 16, 256),
    (8, 8, (700, 300), 0, 128),                       # MHA, S = 6: two splits a group
    (64, 8, (9000, 2049, 1), 16, 256),                # G = 8
    (16, 4, (5000,), 0, 64),                          # S = 79: groups of four, the last one short
]


def _fused_inputs(Hq, Hkv, lens, page, split, dtype="bf16", d=128, **kw):
    base = synth.Workload("fused", B=1, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, split=split, N=1, page_size=page, **kw)
    return synth.make_inputs(synth.with_lens(base, lens))


def _counters_zero(ws):
    import decode_attention_attn_amd as fd
    t = ft.torch()
    t.cuda.synchronize()
    return bool((ws[:fd.TICKET_BYTES] == 0).all().item())


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
@pytest.mark.parametrize("Hq,Hkv,lens,page,split", FUSED_CASES)
def test_fused_merge_matches_the_oracle(Hq, Hkv, lens, page, split, kernel):
    import decode_attention_attn_amd as fd
    inp = _fused_inputs(Hq, Hkv, lens, page, split)
    r = Run(inp)
    ws = fd.alloc_workspace(r.desc(merge="fused", kernel=kernel))
    res = r.run(full=True, workspace=ws, merge="fused", kernel=kernel)
    what = f"fused {kernel} Hq={Hq} Hkv={Hkv} page={page} split={split}"
    e1, e2 = ft.check_exact(res, inp, what=what)
    say(f"[fused] {what}: max|out err|={e1:.3e} max|lse err|={e2:.3e}")
    assert _counters_zero(ws), "a completed call must leave the merge counters zero"
    for b, n in enumerate(lens):
        if n == 0:
            rows = slice(b * Hq, (b + 1) * Hq)
            assert np.all(res["out"][rows] == 0.0) and np.all(res["lse"][rows] == -np.inf)
    # the separate merge gives the same result within the bar
    sep = r.run(full=True, merge="separate", kernel=kernel)
    ft.assert_close(res["out"], sep["out"], inp.w.dtype, what + " vs separate out")
    ft.assert_close(res["lse"], sep["lse"], inp.w.dtype, what + " vs separate lse")


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_fused_merge_workspace_reused_across_inputs(kernel):
    """One workspace for a sequence of different calls: stale partials or
    counters from a previous call would corrupt the next one."""
    import decode_attention_attn_amd as fd
    t = ft.torch()
    ws = t.zeros(64 << 20, dtype=t.uint8, device="cuda")
    cases = [(32, 8, (8000, 3000), 0, 256), (16, 4, (300, 5000, 1200), 16, 256), (32, 8, (8000, 3000), 0, 256),
             (8, 8, (100,), 0, 64)]
    for i, (Hq, Hkv, lens, page, split) in enumerate(cases):
        inp = _fused_inputs(Hq, Hkv, lens, page, split)
        if i == 2:     # the first shape again, other values
            inp.q[:] = synth.normal(99, inp.q.shape, "bf16")
        res = Run(inp).run(full=True, workspace=ws, merge="fused", kernel=kernel)
        ft.check_exact(res, inp, what=f"call {i}")
        assert _counters_zero(ws)


def test_fused_merge_is_bitwise_repeatable():
    inp = _fused_inputs(64, 8, (9000, 2049, 1), 16, 256)
    r = Run(inp)
    first = r.run(full=True, merge="fused")
    for _ in range(4):
        again = r.run(full=True, merge="fused")
        assert np.array_equal(again["raw_out"], first["raw_out"]) and np.array_equal(again["lse"], first["lse"])


@pytest.mark.parametrize("page", [0, 16])
@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_fused_merge_unified_max(kernel, page):
    inp = _fused_inputs(32, 4, (4096, 1500), page, 256, stress_frac=0.02, stress_scale=8.0)
    w = inp.w
    S = -(-w.N // w.split)
    phi, lo, hi = -12.0, -12.0, 12.0
    res = Run(inp).run(full=True, merge="fused", kernel=kernel, mode="unified", phi=phi, lo=lo, hi=hi)
    must, may = ft.flag_bounds(inp, w.split, S, phi, lo, hi)
    got = res["flags"].astype(bool)
    assert np.all(got[must]) and not np.any(got[~may])
    assert res["count"] == int(got.sum()) and 0 < got.sum() < got.size
    ft.check_exact(res, inp, what=f"fused unified {kernel} page={page}")


@pytest.mark.parametrize("q_len,Hq,Hkv", [(4, 32, 8), (8, 32, 8), (3, 16, 4)])
def test_fused_merge_several_query_tokens(q_len, Hq, Hkv):
    base = synth.Workload("fusedmq", B=1, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", split=128, N=1, q_len=q_len)
    inp = synth.make_inputs(synth.with_lens(base, (1000, 129, 3, 2 * q_len)))
    res = Run(inp).run(full=True, merge="fused")
    ft.check_exact(res, inp, what=f"fused q_len={q_len}")


@pytest.mark.parametrize("dtype,d", [("f16", 128), ("f32", 64), ("bf16", 64)])
def test_fused_merge_dtypes(dtype, d):
    inp = _fused_inputs(16, 4, (3000, 1, 700), 0, 128, dtype=dtype, d=d)
    res = Run(inp).run(full=True, merge="fused")
    ft.check_exact(res, inp, what=f"fused {dtype} d={d}")


@pytest.mark.parametrize("name", ["long_gqa_32k", "paged_batched_gqa"])
def test_fused_merge_full_size(name):
    w = synth.WORKLOADS[name]
    say(f"[fused {name}] generating")
    inp = synth.make_inputs(w)
    res = Run(inp).run(full=not w.page_size, merge="fused")
    e1, e2 = ft.check_exact(res, inp, what=f"fused {name}")
    say(f"[fused {name}] every row: max|out err|={e1:.3e} max|lse err|={e2:.3e}")
