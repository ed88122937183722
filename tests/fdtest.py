"""Shared helpers of the GPU tests: upload synth inputs, run the library
through its C ABI, and compare with the fp64 oracle under the stated bar.

Tolerances (elementwise |got - ref| <= atol + rtol * |ref|, reference in fp64):
  fp16 / bf16 cache with fp32 accumulation: atol 2e-3, rtol 1e-2
  fp32 cache: atol 1e-5, rtol 1e-5
  8-bit (E4M3) cache: as 16-bit caches (the values are exact; q is bf16 and
  the accumulation fp32)
Block-table indexing is checked bit-exactly elsewhere (permutation tests).
"""
from __future__ import annotations

import sys

import numpy as np

import decode_attention_attn_amd as fd
import oracle
import synth

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2), "fp8": (2e-3, 1e-2)}
# scores within this distance of a unified-max bound may round to either side
FLAG_MARGIN = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def to_dev(a, dtype):
    t = torch()
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return t.from_numpy(a.view(np.int16)).to("cuda").view(t.bfloat16)
    return t.from_numpy(a).to("cuda")


def f64(x):
    return x.float().cpu().numpy().astype(np.float64)


def raw_numpy(x):
    """Exact storage of a device tensor as numpy (bf16 as uint16 bits)."""
    t = torch()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def assert_close(got, ref, dtype, what, atol=None, rtol=None):
    a, r = TOL[dtype]
    atol = a if atol is None else atol
    rtol = r if rtol is None else rtol
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    both_inf = np.isinf(ref) & (got == ref)
    with np.errstate(invalid="ignore"):          # inf - inf where both are -inf: masked below
        err = np.where(both_inf, 0.0, np.abs(got - ref))
    bound = atol + rtol * np.where(np.isinf(ref), 0.0, np.abs(ref))
    bad = ~(err <= bound)
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside atol={atol} rtol={rtol}; "
                             f"max err {np.nanmax(np.where(np.isfinite(err), err, np.nan)):.3e}; first at {idx}: "
                             f"got {got[idx]!r} ref {ref[idx]!r}")
    return float(np.max(err)) if err.size else 0.0


class Run:
    """Device copies of one synth.Inputs bundle plus the calls on them."""

    def __init__(self, inp: synth.Inputs):
        self.inp = inp
        w = inp.w
        self.w = w
        self.q = to_dev(inp.q, w.q_dtype)
        self.k = to_dev(inp.k, w.dtype)
        self.v = to_dev(inp.v, w.dtype)
        t = torch()
        self.lens = t.from_numpy(inp.seq_lens).to("cuda")
        self.table = t.from_numpy(inp.block_table).to("cuda") if inp.block_table is not None else None

    def desc(self, split=None, mode="sync", phi=0.0, lo=0.0, hi=0.0, kernel="auto", out_dtype=None,
             max_splits=None, merge="auto", fallback="split"):
        w = self.w
        split = split or w.split
        f8 = {}
        if w.dtype == "fp8":
            f8 = dict(q_dtype=w.q_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
            t = torch()
            if w.k_scales is not None:
                self._ks = t.tensor(w.k_scales, dtype=t.float32, device="cuda")
                f8["k_scales"] = self._ks
            if w.v_scales is not None:
                self._vs = t.tensor(w.v_scales, dtype=t.float32, device="cuda")
                f8["v_scales"] = self._vs
        return fd.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, out_dtype, split_size=split,
                            max_splits=max_splits or max(1, -(-w.N // split)), mode=mode, phi=phi, lo=lo,
                            hi=hi, kernel=kernel, q_len=w.q_len, merge=merge, fallback=fallback, **f8)

    def run(self, use_lens=True, full=False, workspace=None, **kw):
        """Partial + combine (contiguous), the paged entry point, or with
        full=True the contiguous fd_decode_attn (merge as kw["merge"] says).
        Returns a dict of float64 numpy results shaped by rows r = b * Hq + h
        (partials are the workspace's when the merge is the single launch)."""
        t = torch()
        w = self.w
        desc = self.desc(**kw)
        S = desc.max_splits
        QR = w.q_len * w.Hq                  # query rows per request
        out = t.empty((w.B, QR, w.d), dtype=fd._tdtype(desc.out_dtype), device="cuda")
        lse = t.empty((w.B, QR), dtype=t.float32, device="cuda")
        flags = t.full((w.B, QR, S), 7, dtype=t.uint8, device="cuda")
        count = t.zeros(1, dtype=t.int32, device="cuda")
        lens = self.lens if use_lens else None
        if w.page_size:
            ws = fd.alloc_workspace(desc) if workspace is None else workspace
            fd.fd_decode_attn_paged(desc, self.q, self.k, self.v, w.page_size, self.table, self.lens, ws, out,
                                    lse, flags, count)
            po, pm, pl = fd.workspace_partials(desc, ws)
        elif full:
            ws = fd.alloc_workspace(desc) if workspace is None else workspace
            fd.fd_decode_attn(desc, self.q, self.k, self.v, w.N, self.lens if use_lens else None, ws, out, lse,
                              flags, count)
            po, pm, pl = fd.workspace_partials(desc, ws)
        else:
            po, pm, pl, _ = fd.alloc_partials(desc)
            fd.fd_decode_attn_partial(desc, self.q, self.k, self.v, w.N, lens, po, pm, pl, flags, count)
            fd.fd_decode_attn_combine(desc, po, pm, pl, lens, out, lse)
        t.cuda.synchronize()
        R = w.B * QR
        return dict(out=f64(out).reshape(R, w.d), lse=f64(lse).reshape(R),
                    part_o=f64(po).reshape(R, S, w.d), part_m=f64(pm).reshape(R, S),
                    part_l=f64(pl).reshape(R, S), flags=flags.cpu().numpy().reshape(R, S),
                    count=int(count.item()), raw_out=raw_numpy(out), desc=desc)


def oracle_exact(inp, rows=None):
    p = oracle.problem_of(inp)
    return oracle.attention(p, inp.q, inp.k, inp.v, seq_lens=inp.seq_lens, block_table=inp.block_table,
                            rows=rows)


def oracle_partials(inp, split, S, rows=None):
    p = oracle.problem_of(inp)
    return oracle.split_partials(p, inp.q, inp.k, inp.v, split, S, seq_lens=inp.seq_lens,
                                 block_table=inp.block_table, rows=rows)


def check_exact(res, inp, rows=None, what=""):
    """out and lse against the oracle's exact attention on `rows` (all if None)."""
    ref, lref = oracle_exact(inp, rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    e1 = assert_close(res["out"][sel], ref[sel], inp.w.dtype, f"{what} out")
    e2 = assert_close(res["lse"][sel], lref[sel], inp.w.dtype, f"{what} lse")
    return e1, e2


def check_partials(res, inp, split, rows=None, what=""):
    S = res["part_m"].shape[1]
    po, pm, pl = oracle_partials(inp, split, S, rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    valid = pl[sel] > 0
    dt = inp.w.dtype
    assert np.array_equal(res["part_l"][sel] > 0, valid), f"{what}: set of non-empty splits differs"
    assert np.all(res["part_m"][sel][~valid] == -np.inf), f"{what}: empty split m must be -inf"
    assert_close(res["part_m"][sel][valid], pm[sel][valid], dt, f"{what} part_m")
    assert_close(res["part_l"][sel][valid], pl[sel][valid], dt, f"{what} part_l")
    assert_close(res["part_o"][sel][valid], po[sel][valid], dt, f"{what} part_o")


def flag_bounds(inp, split, S, phi, lo, hi, rows=None):
    """(must_flag, may_flag) from the oracle with the bounds moved in and out by
    FLAG_MARGIN: a GPU flag set F is valid iff must <= F <= may."""
    p = oracle.problem_of(inp)
    kw = dict(seq_lens=inp.seq_lens, block_table=inp.block_table, rows=rows)
    must = oracle.unified_max(p, inp.q, inp.k, inp.v, split, S, phi, lo - FLAG_MARGIN, hi + FLAG_MARGIN, **kw)
    may = oracle.unified_max(p, inp.q, inp.k, inp.v, split, S, phi, lo + FLAG_MARGIN, hi - FLAG_MARGIN, **kw)
    return must["flags"].astype(bool), may["flags"].astype(bool)


def sample_rows(w, n, seed=0):
    R = w.B * w.q_len * w.Hq
    if n >= R:
        return np.arange(R, dtype=np.int32)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(R, size=n, replace=False)).astype(np.int32)
