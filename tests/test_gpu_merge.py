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
