"""fd_decode_attn_paged_noalloc: the paged entry point without a workspace.

Its partials live in the library's per-GPU scratch array.  Two calls in a
row (the second smaller, so the array still holds the first call's partials
beyond what the second writes) must each give the bits of
fd_decode_attn_paged with a workspace of its own, and the oracle's values.
A shape whose partials exceed the array is refused.
"""
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


def _both(inp, **kw):
    """(workspace result, no-alloc result) as dicts of numpy arrays."""
    import decode_attention_attn_amd as fd
    t = ft.torch()
    r = Run(inp)
    w = inp.w
    desc = r.desc(**kw)
    res = []
    for noalloc in (False, True):
        out = t.full((w.B, w.Hq, w.d), 3.0, dtype=fd._tdtype(desc.out_dtype), device="cuda")
        lse = t.full((w.B, w.Hq), 3.0, dtype=t.float32, device="cuda")
        flags = t.full((w.B, w.Hq, desc.max_splits), 7, dtype=t.uint8, device="cuda")
        count = t.zeros(1, dtype=t.int32, device="cuda")
        if noalloc:
            fd.fd_decode_attn_paged_noalloc(desc, r.q, r.k, r.v, w.page_size, r.table, r.lens, out, lse, flags,
                                            count)
        else:
            fd.fd_decode_attn_paged(desc, r.q, r.k, r.v, w.page_size, r.table, r.lens, fd.alloc_workspace(desc),
                                    out, lse, flags, count)
        t.cuda.synchronize()
        R = w.B * w.Hq
        res.append(dict(out=ft.f64(out).reshape(R, w.d), lse=ft.f64(lse).reshape(R),
                        raw=ft.raw_numpy(out), flags=flags.cpu().numpy(), count=int(count.item())))
    return res


def _check_pair(inp, what, **kw):
    ws, na = _both(inp, **kw)
    assert np.array_equal(na["raw"], ws["raw"]), f"{what}: out differs from the workspace call"
    assert np.array_equal(na["lse"], ws["lse"]), f"{what}: lse differs from the workspace call"
    assert np.array_equal(na["flags"], ws["flags"]) and na["count"] == ws["count"], what
    e1, e2 = ft.check_exact(na, inp, what=what)
    say(f"[no-alloc] {what}: max|out err|={e1:.3e} max|lse err|={e2:.3e}")


def test_noalloc_two_calls_second_smaller():
    big = synth.Workload("na_big", B=4, Hq=32, Hkv=8, d=128, dtype="bf16", split=256, N=1, page_size=16)
    small = synth.Workload("na_small", B=2, Hq=16, Hkv=4, d=64, dtype="bf16", split=128, N=1, page_size=16)
    _check_pair(synth.make_inputs(synth.with_lens(big, (5000, 1200, 3333, 17))), "first call")
    _check_pair(synth.make_inputs(synth.with_lens(small, (700, 300))), "second, smaller call")


def test_noalloc_unified_max_matches_the_workspace_call():
    base = synth.Workload("na_umax", B=2, Hq=32, Hkv=4, d=128, dtype="bf16", split=256, N=1, page_size=16,
                          stress_frac=0.02, stress_scale=8.0)
    inp = synth.make_inputs(synth.with_lens(base, (4096, 1500)))
    _check_pair(inp, "unified max", mode="unified", phi=-12.0, lo=-12.0, hi=12.0)


def test_noalloc_refuses_partials_larger_than_its_array():
    import ctypes as C
    import decode_attention_attn_amd as fd
    # 64 requests x 64 query heads x 64 splits x 128 dims of fp32: 128 MiB of partials
    desc = fd.make_desc(64, 64, 8, 128, "bf16", split_size=256, max_splits=64)
    assert fd.fd_workspace_bytes(desc) > fd.NOALLOC_SCRATCH_BYTES
    st = fd.lib().fd_decode_attn_paged_noalloc(C.byref(desc), None, None, None, 1, 16, None, 1, None, None,
                                               None, None, None, None)
    assert st == fd.FD_ERR_WORKSPACE_TOO_SMALL
