"""The C ABI on streams other than the default one, and under HIP graph capture.

The library enqueues every kernel on the stream it is given and allocates,
clears and synchronises nothing itself, so a call on a side stream gives the
same bits as on the default stream, and a captured call replays like an eager
one.  The graph cases replay several times with new query values copied into
the same buffer between replays, with eager work in between, and compare every
replay bit for bit with an eager call on the same values (and one replay with
the oracle).
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


def _inputs(page, q_len=1, split=256, dtype="bf16"):
    base = synth.Workload("streams", B=3, Hq=32, Hkv=8, d=128, dtype=dtype, split=split, N=1, page_size=page,
                          q_len=q_len)
    return synth.make_inputs(synth.with_lens(base, [4100, 517, 2049]))


# (page size, entry point) cases: partial + combine, the paged entry point
# (AUTO), the contiguous fd_decode_attn with the single-launch merge (its
# counters must come back to zero on every replay), a one-split call of 40
# query tokens per request (query tiles sharing K and V, the result written
# by the partial kernel), and an fp32 cache under AUTO (the VALU kernel's
# single launch, 5 splits)
CASES = {"partial+combine": (0, "separate", 1, 256, "bf16"), "paged": (16, "auto", 1, 256, "bf16"),
         "single launch": (0, "fused", 1, 256, "bf16"), "tiles, direct": (0, "auto", 40, 8192, "bf16"),
         "fp32, VALU single launch": (0, "auto", 1, 1024, "f32")}


class _Call:
    """One decode call on fixed buffers: partial + combine, the paged entry
    point, or the contiguous entry point with its merge mode."""

    def __init__(self, r: Run, merge="separate"):
        import decode_attention_attn_amd as fd
        t = ft.torch()
        self.fd, self.r, w = fd, r, r.w
        self.merge = merge
        self.desc = r.desc(merge=merge)
        self.out = t.empty((w.B, w.q_len * w.Hq, w.d), dtype=fd._tdtype(self.desc.out_dtype), device="cuda")
        self.lse = t.empty((w.B, w.q_len * w.Hq), dtype=t.float32, device="cuda")
        if w.page_size or merge != "separate":
            self.ws = fd.alloc_workspace(self.desc)
        else:
            self.po, self.pm, self.pl, _ = fd.alloc_partials(self.desc)

    def __call__(self, stream=None):
        fd, r, w = self.fd, self.r, self.r.w
        if w.page_size:
            fd.fd_decode_attn_paged(self.desc, r.q, r.k, r.v, w.page_size, r.table, r.lens, self.ws, self.out,
                                    self.lse, stream=stream)
        elif self.merge != "separate":
            fd.fd_decode_attn(self.desc, r.q, r.k, r.v, w.N, r.lens, self.ws, self.out, self.lse, stream=stream)
        else:
            fd.fd_decode_attn_partial(self.desc, r.q, r.k, r.v, w.N, r.lens, self.po, self.pm, self.pl,
                                      stream=stream)
            fd.fd_decode_attn_combine(self.desc, self.po, self.pm, self.pl, r.lens, self.out, self.lse,
                                      stream=stream)

    def result(self):
        w = self.r.w
        R = w.B * w.q_len * w.Hq
        return ft.f64(self.out).reshape(R, w.d), ft.f64(self.lse).reshape(R)


@pytest.mark.parametrize("page", [0, 16])
def test_side_stream_gives_the_default_stream_bits(page):
    t = ft.torch()
    inp = _inputs(page)
    call = _Call(Run(inp))
    call()
    t.cuda.synchronize()
    ref_out, ref_lse = call.result()
    call.out.fill_(0)
    call.lse.fill_(0)
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        call(stream=side)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    out, lse = call.result()
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)
    ft.check_exact(dict(out=out, lse=lse), inp, what=f"side stream page={page}")


@pytest.mark.parametrize("case", list(CASES))
def test_captured_call_replays_like_eager(case):
    t = ft.torch()
    page, merge, q_len, split, dtype = CASES[case]
    inp = _inputs(page, q_len, split, dtype)
    r = Run(inp)
    call = _Call(r, merge)
    w = inp.w
    qs = [synth.normal(900 + i, inp.q.shape, w.q_dtype) for i in range(3)]

    # warm up on a side stream, then capture one call
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        call()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        call()
    t.cuda.synchronize()

    for i, qi in enumerate(qs):
        r.q.copy_(ft.to_dev(qi, w.q_dtype))
        call()                                   # eager on the same buffers
        t.cuda.synchronize()
        ref_out, ref_lse = call.result()
        call.out.fill_(0)
        call.lse.fill_(0)
        graph.replay()
        t.cuda.synchronize()
        out, lse = call.result()
        say(f"[graph {case}] replay {i}: max|out - eager| = {np.abs(out - ref_out).max():.3e}")
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse), f"replay {i}"
        if i == len(qs) - 1:
            ft.check_exact(dict(out=out, lse=lse), synth.Inputs(w, qi, inp.k, inp.v, inp.seq_lens,
                                                                inp.block_table), what=f"graph {case}")
