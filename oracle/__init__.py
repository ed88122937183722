"""ctypes wrapper of the fp64 decode-attention oracle (oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg import this module.  It shares no code with the GPU library
(decode_attention_attn_amd) and neither imports the other.  Arguments are
numpy arrays in the storage conventions of the `synth` module (f32 -> float32,
f16 -> float16, bf16 -> uint16 bit patterns, fp8 (OCP E4M3, K and V only) ->
uint8 bit patterns); results are float64.

The arithmetic and its citations are in oracle.c; this file only marshals.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SRC = _HERE / "oracle.c"
LIB = _HERE / "liboracle.so"
BUILD_CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
             str(SRC), "-o", str(LIB), "-lm"]

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
_NAME = {v: k for k, v in DTYPE_CODE.items()}
_NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}


class OracleProblem(C.Structure):
    _fields_ = [("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("d", C.c_int32),
                ("dtype", C.c_int32), ("N", C.c_int32), ("page_size", C.c_int32),
                ("max_blocks", C.c_int32), ("scale", C.c_double), ("q_dtype", C.c_int32),
                ("k_scale", C.c_double), ("v_scale", C.c_double), ("q_len", C.c_int32),
                ("k_scales", C.c_void_p), ("v_scales", C.c_void_p)]


def build() -> Path:
    subprocess.run(BUILD_CMD, check=True)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        L = C.CDLL(str(LIB))
        vp, i32p = C.c_void_p, C.POINTER(C.c_int32)
        dp = C.POINTER(C.c_double)
        pp = C.POINTER(OracleProblem)
        L.oracle_attention.argtypes = [pp, vp, vp, vp, i32p, i32p, i32p, C.c_int, C.c_int, dp, dp]
        L.oracle_split_partials.argtypes = [pp, vp, vp, vp, i32p, i32p, C.c_int, C.c_int, i32p, C.c_int,
                                            C.c_int, dp, dp, dp]
        L.oracle_merge.argtypes = [C.c_int, C.c_int, C.c_int, dp, dp, dp, dp, dp]
        L.oracle_merge_lse.argtypes = [C.c_int, C.c_int, C.c_int, dp, dp, dp, dp, dp]
        L.oracle_online_tiles.argtypes = [C.c_int, C.c_int, dp, dp, C.c_int, dp, dp, dp, dp, dp]
        L.oracle_out_of_range.argtypes = [C.c_double, C.c_double, C.c_double]
        L.oracle_unified_max.argtypes = [pp, vp, vp, vp, i32p, i32p, C.c_int, C.c_int, C.c_double, C.c_double,
                                         C.c_double, i32p, C.c_int, C.c_int, dp, dp, dp,
                                         C.POINTER(C.c_uint8), dp, dp, C.POINTER(C.c_longlong), C.c_int]
        L.oracle_decode.argtypes = [C.c_int, vp, C.c_size_t, dp]
        for f in ("oracle_attention", "oracle_split_partials", "oracle_merge", "oracle_merge_lse",
                  "oracle_online_tiles", "oracle_out_of_range", "oracle_unified_max"):
            getattr(L, f).restype = C.c_int
        L.oracle_decode.restype = None
        _lib = L
    return _lib


def host_cpus() -> dict:
    """What the host offers this process: every CPU it has (nproc), those the
    process may run on (its affinity mask), and the OpenMP thread limit the
    environment sets, if any."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    limit = os.environ.get("OMP_NUM_THREADS", "")
    return {"nproc": os.cpu_count() or 1, "affinity": affinity,
            "omp_num_threads": int(limit) if limit.isdigit() and int(limit) > 0 else None}


def default_threads() -> int:
    """One thread per CPU the process may run on, within OMP_NUM_THREADS when
    the environment sets it (a shared host's allotment to this process)."""
    c = host_cpus()
    n = c["affinity"]
    if c["omp_num_threads"]:
        n = min(n, c["omp_num_threads"])
    return max(1, n)


# ----------------------------------------------------------------------------
def _ptr(a, ctype):
    return a.ctypes.data_as(C.POINTER(ctype)) if a is not None else None


def _vp(a):
    return C.c_void_p(a.ctypes.data) if a is not None else None


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle returned {rc}")


def _storage(a, dtype):
    a = np.ascontiguousarray(a)
    want = _NP_STORAGE[dtype]
    if a.dtype != want:
        raise TypeError(f"expected {want} storage for {dtype}, got {a.dtype}")
    return a


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def problem(B, Hq, Hkv, d, dtype, N=0, page_size=0, max_blocks=0, scale=None, q_dtype=None, k_scale=1.0,
            v_scale=1.0, q_len=1, k_scales=None, v_scales=None):
    """dtype: storage of K and V; q_dtype: storage of q (default: dtype; bf16 for fp8 caches);
    q_len query tokens per request (q [B, q_len, Hq, d]; results by row (b*q_len + i)*Hq + h).
    k_scales / v_scales: per-KV-head scales [Hkv] replacing k_scale / v_scale."""
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if q_dtype is None:
        q_dtype = "bf16" if dtype == "fp8" else dtype
    p = OracleProblem(B, Hq, Hkv, d, DTYPE_CODE[dtype], N, page_size, max_blocks, float(scale),
                      DTYPE_CODE[q_dtype], float(k_scale), float(v_scale), int(q_len), None, None)
    keep = []
    for name, arr in (("k_scales", k_scales), ("v_scales", v_scales)):
        if arr is not None:
            a = np.ascontiguousarray(arr, dtype=np.float64)
            if a.shape != (Hkv,):
                raise ValueError(f"{name} must have shape ({Hkv},)")
            keep.append(a)
            setattr(p, name, a.ctypes.data)
    p._keep = keep          # the arrays live as long as the problem
    return p


def problem_of(inp, scale=None):
    """OracleProblem for a synth.Inputs bundle."""
    w = inp.w
    return problem(w.B, w.Hq, w.Hkv, w.d, w.dtype, N=w.N, page_size=w.page_size,
                   max_blocks=w.max_blocks if w.page_size else 0, scale=scale, q_dtype=w.q_dtype,
                   k_scale=w.k_scale, v_scale=w.v_scale, q_len=w.q_len,
                   k_scales=getattr(w, "k_scales", None), v_scales=getattr(w, "v_scales", None))


def _nrows(p):
    return p.B * p.q_len * p.Hq


def _rows_arg(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int32)
    return r, int(r.size)


def attention(p, q, k, v, seq_lens=None, block_table=None, rows=None, threads=None):
    """Exact attention.  Returns (out [B*Hq, d], lse [B*Hq]) as float64; rows not
    selected are NaN."""
    dtype = _NAME[p.dtype]
    q, k, v = _storage(q, _NAME[p.q_dtype]), _storage(k, dtype), _storage(v, dtype)
    sl, bt = _i32(seq_lens), _i32(block_table)
    r, nr = _rows_arg(rows)
    out = np.full((_nrows(p), p.d), np.nan)
    lse = np.full(_nrows(p), np.nan)
    rc = lib().oracle_attention(C.byref(p), _vp(q), _vp(k), _vp(v), _ptr(sl, C.c_int32), _ptr(bt, C.c_int32),
                                _ptr(r, C.c_int32), nr, threads or default_threads(),
                                _ptr(out, C.c_double), _ptr(lse, C.c_double))
    _check(rc, "oracle_attention")
    return out, lse


def split_partials(p, q, k, v, split, S_max, seq_lens=None, block_table=None, rows=None, threads=None):
    """Per-split (O_s normalised, m_s, l_s): shapes [B*Hq, S_max, d], [B*Hq, S_max] x2."""
    dtype = _NAME[p.dtype]
    q, k, v = _storage(q, _NAME[p.q_dtype]), _storage(k, dtype), _storage(v, dtype)
    sl, bt = _i32(seq_lens), _i32(block_table)
    r, nr = _rows_arg(rows)
    R = _nrows(p)
    po = np.full((R, S_max, p.d), np.nan)
    pm = np.full((R, S_max), np.nan)
    pl = np.full((R, S_max), np.nan)
    rc = lib().oracle_split_partials(C.byref(p), _vp(q), _vp(k), _vp(v), _ptr(sl, C.c_int32),
                                     _ptr(bt, C.c_int32), split, S_max, _ptr(r, C.c_int32), nr,
                                     threads or default_threads(), _ptr(po, C.c_double),
                                     _ptr(pm, C.c_double), _ptr(pl, C.c_double))
    _check(rc, "oracle_split_partials")
    return po, pm, pl


def merge(part_o, part_m, part_l, form="max"):
    """Merge partials [R, S, d], [R, S], [R, S] -> (out [R, d], lse [R])."""
    po = np.ascontiguousarray(part_o, dtype=np.float64)
    pm = np.ascontiguousarray(part_m, dtype=np.float64)
    pl = np.ascontiguousarray(part_l, dtype=np.float64)
    R, S, d = po.shape
    out = np.empty((R, d))
    lse = np.empty(R)
    fn = lib().oracle_merge if form == "max" else lib().oracle_merge_lse
    _check(fn(R, S, d, _ptr(po, C.c_double), _ptr(pm, C.c_double), _ptr(pl, C.c_double),
              _ptr(out, C.c_double), _ptr(lse, C.c_double)), "oracle_merge")
    return out, lse


def online_tiles(scores, v, tile):
    """FlashAttention tile recurrence over one row.  scores [n], v [n, d].
    Returns (out [d], lse, trace_m [T], trace_l [T], trace_acc [T, d])."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    vv = np.ascontiguousarray(v, dtype=np.float64)
    n, d = vv.shape
    T = -(-n // tile)
    tm, tl, ta = np.empty(T), np.empty(T), np.empty((T, d))
    out = np.empty(d)
    lse = C.c_double()
    _check(lib().oracle_online_tiles(n, d, _ptr(s, C.c_double), _ptr(vv, C.c_double), tile,
                                     _ptr(tm, C.c_double), _ptr(tl, C.c_double), _ptr(ta, C.c_double),
                                     _ptr(out, C.c_double), C.byref(lse)), "oracle_online_tiles")
    return out, lse.value, tm, tl, ta


def out_of_range(s, lo, hi) -> bool:
    return bool(lib().oracle_out_of_range(float(s), float(lo), float(hi)))


def unified_max(p, q, k, v, split, S_max, phi, lo, hi, seq_lens=None, block_table=None, rows=None,
                threads=None, whole_row=False):
    """Unified-max softmax with fallback: per split, or with whole_row every
    split of a row that has a flagged split.  Returns a dict with out, lse,
    part_o/part_m/part_l, flags [B*Hq, S_max] (uint8: the splits whose scores
    left the range) and n_flagged."""
    dtype = _NAME[p.dtype]
    q, k, v = _storage(q, _NAME[p.q_dtype]), _storage(k, dtype), _storage(v, dtype)
    sl, bt = _i32(seq_lens), _i32(block_table)
    r, nr = _rows_arg(rows)
    R = _nrows(p)
    po = np.full((R, S_max, p.d), np.nan)
    pm = np.full((R, S_max), np.nan)
    pl = np.full((R, S_max), np.nan)
    fl = np.zeros((R, S_max), dtype=np.uint8)
    out = np.full((R, p.d), np.nan)
    lse = np.full(R, np.nan)
    nf = C.c_longlong(0)
    rc = lib().oracle_unified_max(C.byref(p), _vp(q), _vp(k), _vp(v), _ptr(sl, C.c_int32), _ptr(bt, C.c_int32),
                                  split, S_max, float(phi), float(lo), float(hi), _ptr(r, C.c_int32), nr,
                                  threads or default_threads(), _ptr(po, C.c_double), _ptr(pm, C.c_double),
                                  _ptr(pl, C.c_double), _ptr(fl, C.c_uint8), _ptr(out, C.c_double),
                                  _ptr(lse, C.c_double), C.byref(nf), int(bool(whole_row)))
    _check(rc, "oracle_unified_max")
    return dict(out=out, lse=lse, part_o=po, part_m=pm, part_l=pl, flags=fl, n_flagged=nf.value)


def decode(a, dtype):
    """Exact float64 values of a storage array, decoded by the oracle's own code."""
    a = _storage(a, dtype)
    out = np.empty(a.size)
    lib().oracle_decode(DTYPE_CODE[dtype], _vp(a), a.size, _ptr(out, C.c_double))
    return out.reshape(a.shape)
