"""Benchmark: split-KV decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole decode-attention pass over one batch: the split-partial
kernel plus the combine kernel.  The default workload is the long-context
GQA decode (B=1, Hq=32, Hkv=8, d=128, N=32768, bf16 cache, split 256).

Inputs are generated once (seeded, synthetic), copied to HBM, and replicated
so that consecutive steps read different copies of the KV cache; the copies
together exceed the 256 MB Infinity Cache, so every step streams its K and V
from HBM.  Timing uses HIP events recorded on the stream the kernels are
launched on (torch's current stream): one pair around the K timed steps
(nothing else runs in between), then one pair around K back-to-back launches
of each kernel alone for the per-kernel averages the roofline uses.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py --summarize-profile DIR   writes profile summaries
        (rocprofv3 kernel-trace stats and PMC counter CSVs under DIR) as
        markdown tables to stdout.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, AMD public spec
MFMA_PEAK_TFLOPS = 2500.0         # MI355X dense bf16 / f16 matrix peak (the 16-bit and 8-bit caches' path)
VALU_F32_PEAK_TFLOPS = 157.3      # MI355X fp32 vector peak (the fp32 cache's VALU kernel)
MALL_BYTES = 256 * 2 ** 20        # Infinity Cache
PARTIAL_KERNEL = "partial"        # substring of the split-partial kernels' names
COPY_BYTES = 256 * 2 ** 20        # calibration copy: reads and writes this many bytes
COMBINE_KERNEL = "combine_kernel"
KERNEL_SOURCES = ["decode_attention_attn_amd/csrc/fd_partial_valu.hip",
                  "decode_attention_attn_amd/csrc/fd_partial_mfma.h",
                  "decode_attention_attn_amd/csrc/fd_device.h",
                  "decode_attention_attn_amd/csrc/fd_merge.h",
                  "decode_attention_attn_amd/csrc/fd_combine.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def default_merge(workload: str, split: int = 0, kernel: str = "auto") -> str:
    """The merge mode a bench run uses unless told: contiguous caches time the
    partial and combine kernels apart (the roofline is the partial kernel's),
    except where the library's AUTO runs one kernel -- one split per row (the
    partial kernel writes the result) and the VALU kernel (fp32 caches) with
    at most 16 splits (its single launch) -- which, like a paged cache, run as
    one call of the library."""
    import synth
    w0 = synth.WORKLOADS[workload]
    n_splits = -(-w0.N // (split or w0.split))
    valu = kernel == "valu" or (kernel == "auto" and w0.dtype == "f32")
    one_kernel = n_splits == 1 or (valu and n_splits <= 16)
    return "auto" if (w0.page_size or one_kernel) else "separate"


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update((ROOT / f).read_bytes())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# algorithmic bytes
# ----------------------------------------------------------------------------
def algorithmic_bytes(inp):
    """Bytes the method must move once: K and V of every (request, KV head,
    valid token), q, the output, and the block-table entries of the valid pages."""
    import synth
    w = inp.w
    eb = synth.ELEM_BYTES[w.dtype]
    qb = synth.ELEM_BYTES[w.q_dtype]       # q and out (out has q's type)
    kv = inp.kv_bytes
    q = w.B * w.q_len * w.Hq * w.d * qb
    out = w.B * w.q_len * w.Hq * w.d * qb
    table = 0
    if w.page_size:
        table = int(((inp.seq_lens.astype(np.int64) + w.page_size - 1) // w.page_size).sum()) * 4
    # flops: q.k and p.v, 2 d each, for every (query row, cache token it sees)
    lens = inp.seq_lens.astype(np.int64)
    seen = np.clip(lens[:, None] - w.q_len + np.arange(w.q_len, dtype=np.int64)[None, :] + 1, 0, lens[:, None])
    flops = 4 * w.d * w.Hq * int(seen.sum())
    return dict(kv=kv, q=q, out=out, table=table, partial=kv + q + table, step=kv + q + out + table,
                units=int(lens.sum()) * w.Hkv, per_unit=2 * w.d * eb, flops=flops)


def roofline_bound(w, kernel, alg):
    """'hbm' or 'mfma'/'valu' for the partial kernel, with the compute peak of
    the kernel that runs it: whichever of the algorithmic bytes at the HBM
    peak and the algorithmic flops at the compute peak takes longer."""
    matrix = w.dtype in ("f16", "bf16", "fp8") and kernel != "valu"
    peak = MFMA_PEAK_TFLOPS if matrix else VALU_F32_PEAK_TFLOPS
    compute_s = alg["flops"] / (peak * 1e12)
    memory_s = alg["partial"] / (HBM_PEAK_GBPS * 1e9)
    if compute_s <= memory_s:
        return "hbm", HBM_PEAK_GBPS
    return ("mfma" if matrix else "valu"), peak


# ----------------------------------------------------------------------------
def run_gpu(args, inp, wl):
    import torch
    import decode_attention_attn_amd as fd

    dev = torch.device("cuda:0")
    w = inp.w
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def dev_t(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q = dev_t(inp.q, w.q_dtype)
    k0, v0 = dev_t(inp.k, w.dtype), dev_t(inp.v, w.dtype)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    table = torch.from_numpy(inp.block_table).to(dev) if w.page_size else None
    kv_bytes = k0.numel() * k0.element_size() * 2
    copies = max(1, math.ceil(4 * MALL_BYTES / kv_bytes)) if not args.warm else 1
    ks, vs = [k0], [v0]
    for _ in range(copies - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    log(f"[bench] {w.name}: {copies} KV copies of {kv_bytes / 2**20:.1f} MiB")

    mode = args.mode
    f8 = dict(q_dtype=w.q_dtype, k_scale=w.k_scale, v_scale=w.v_scale) if w.dtype == "fp8" else {}
    if w.dtype == "fp8" and w.k_scales is not None:
        f8["k_scales"] = torch.tensor(w.k_scales, dtype=torch.float32, device=dev)
    if w.dtype == "fp8" and w.v_scales is not None:
        f8["v_scales"] = torch.tensor(w.v_scales, dtype=torch.float32, device=dev)
    desc = fd.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, split_size=w.split, max_seq_len=w.N, mode=mode,
                        phi=args.phi, lo=args.lo, hi=args.hi, kernel=args.kernel, q_len=w.q_len, merge=args.merge,
                        fallback=args.fallback, **f8)
    S = desc.max_splits
    out = torch.empty((w.B, w.q_len * w.Hq, w.d), dtype=fd._tdtype(desc.out_dtype), device=dev)
    lse = torch.empty((w.B, w.q_len * w.Hq), dtype=torch.float32, device=dev)
    flags = torch.zeros((w.B, w.q_len * w.Hq, S), dtype=torch.uint8, device=dev) if mode == "unified" else None
    count = torch.zeros(1, dtype=torch.int32, device=dev) if mode == "unified" else None
    L = fd.lib()
    stream = torch.cuda.current_stream()
    sp = fd._stream(stream)
    import ctypes as C
    dref = C.byref(desc)

    if w.page_size:
        ws = fd.alloc_workspace(desc, dev)
        # the paged entry point does partial and merge; time it as one, the kernels split in rocprof
        calls = []
        for i in range(copies):
            calls.append(lambda i=i: fd.fd_decode_attn_paged(desc, q, ks[i], vs[i], w.page_size, table, lens, ws,
                                                             out, lse, flags, count, stream))
        combine = None
    elif args.merge != "separate":
        # fd_decode_attn: partial and merge in one call (one launch when the merge is fused)
        ws = fd.alloc_workspace(desc, dev)
        fd.fd_decode_attn(desc, q, ks[0], vs[0], w.N, lens, ws, out, lse, flags, count, stream)
        vp = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
        fargs = [(dref, vp(q), vp(ks[i]), vp(vs[i]), C.c_int32(w.N), vp(lens), vp(ws), C.c_size_t(ws.numel()),
                  vp(out), vp(lse), vp(flags), vp(count), sp) for i in range(copies)]
        full_fn = L.fd_decode_attn

        def check_full(st):
            if st != 0:
                raise RuntimeError(f"fd_decode_attn: {fd.fd_status_string(st)}")

        calls = [lambda i=i: check_full(full_fn(*fargs[i])) for i in range(copies)]
        combine = None
    else:
        po, pm, pl, _ = fd.alloc_partials(desc, dev)
        # validate the marshalling once through the binding, then call the C entry
        # points with the same prepared arguments in the timed loop
        fd.fd_decode_attn_partial(desc, q, ks[0], vs[0], w.N, lens, po, pm, pl, flags, count, stream)
        fd.fd_decode_attn_combine(desc, po, pm, pl, lens, out, lse, stream)
        vp = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
        pargs = [(dref, vp(q), vp(ks[i]), vp(vs[i]), C.c_int32(w.N), vp(lens), vp(po), vp(pm), vp(pl), vp(flags),
                  vp(count), sp) for i in range(copies)]
        cargs = (dref, vp(po), vp(pm), vp(pl), vp(lens), vp(out), vp(lse), sp)
        part_fn, comb_fn = L.fd_decode_attn_partial, L.fd_decode_attn_combine

        def check(st, name):
            if st != 0:
                raise RuntimeError(f"{name}: {fd.fd_status_string(st)}")

        calls = [lambda i=i: check(part_fn(*pargs[i]), "partial") for i in range(copies)]
        combine = lambda: check(comb_fn(*cargs), "combine")

    for i in range(args.warmup):
        calls[i % copies]()
        if combine:
            combine()
    torch.cuda.synchronize()

    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(body, n):
        """Average ms of body() over n back-to-back runs, HIP events on `stream`."""
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            body(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def step(i):
        calls[i % copies]()
        if combine:
            combine()

    # the timed steps: K whole steps, nothing else in between
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    if args.graph:
        # one HIP graph holding one step per KV copy, captured through the
        # binding on torch's capture stream and replayed K / copies times
        def bind_step(i):
            if w.page_size:
                fd.fd_decode_attn_paged(desc, q, ks[i], vs[i], w.page_size, table, lens, ws, out, lse, flags, count)
            else:
                fd.fd_decode_attn_partial(desc, q, ks[i], vs[i], w.N, lens, po, pm, pl, flags, count)
                fd.fd_decode_attn_combine(desc, po, pm, pl, lens, out, lse)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(copies):
                bind_step(i)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(1, K // copies)
        t_wall = time.perf_counter()
        step_ms = timed(lambda i: graph.replay(), reps) / copies
        K = reps * copies
    else:
        step_ms = timed(step, K)
    t_wall = time.perf_counter() - t_wall
    # per-kernel averages: K back-to-back launches of each kernel alone
    part_ms = timed(lambda i: calls[i % copies](), K)
    comb_ms = timed(lambda i: combine(), K) if combine else 0.0
    part_us = np.array([part_ms * 1e3])
    comb_us = np.array([comb_ms * 1e3])

    # one step's result, for the parity spot check
    calls[0]()
    if combine:
        combine()
    torch.cuda.synchronize()
    res = dict(out=out.float().cpu().numpy().reshape(-1, w.d).astype(np.float64),
               lse=lse.cpu().numpy().reshape(-1).astype(np.float64),
               flags=flags.cpu().numpy() if flags is not None else None)
    return dict(step_ms=step_ms, wall_ms=t_wall * 1e3 / K, part_us=part_us, comb_us=comb_us, copies=copies,
                res=res, S=S, device=torch.cuda.get_device_name(0), steps=K)


def fallback_stats(inp, flags, args):
    """Flagged (request, query head, split) triples of the last step, out of those
    that hold tokens; each flagged one was recomputed with the synchronized softmax
    (with the whole-row fallback: every split of a row with a flagged split)."""
    w = inp.w
    S = flags.shape[-1]
    lens = inp.seq_lens.astype(np.int64)[:, None]
    causal = np.clip(lens - w.q_len + np.arange(w.q_len)[None, :] + 1, 0, lens)   # tokens each query row sees
    per_row = np.repeat(np.minimum(-(-causal // w.split), S).reshape(-1), w.Hq)   # splits with tokens, by row
    valid = int(per_row.sum())
    n = int(flags.astype(np.int64).sum())
    rows_flagged = flags.reshape(-1, S).astype(bool).any(axis=1)
    out = {"flagged_splits": n, "splits_with_tokens": valid, "rate": n / max(valid, 1), "fallback": args.fallback,
           "phi": args.phi, "lo": args.lo, "hi": args.hi}
    if args.fallback == "row":
        out["rows_flagged"] = int(rows_flagged.sum())
        out["recomputed_splits"] = int(per_row[rows_flagged].sum())
    return out


def parity_spot_check(inp, res, rows):
    import oracle
    p = oracle.problem_of(inp)
    ref, lref = oracle.attention(p, inp.q, inp.k, inp.v, seq_lens=inp.seq_lens, block_table=inp.block_table,
                                 rows=rows)
    tol = {"f32": (1e-5, 1e-5)}.get(inp.w.dtype, (2e-3, 1e-2))
    e = np.abs(res["out"][rows] - ref[rows])
    el = np.abs(res["lse"][rows] - lref[rows])
    ok = bool(np.all(e <= tol[0] + tol[1] * np.abs(ref[rows])) and np.all(el <= tol[0] + tol[1] * np.abs(lref[rows])))
    return dict(rows=int(len(rows)), max_abs_err_out=float(e.max()), max_abs_err_lse=float(el.max()), ok=ok)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, alg, seconds):
    """The fp64 oracle, as it is, on the host cores: whole decode steps of the
    same workload repeated until about `seconds` of work have run, on one
    thread per CPU the process may use (within OMP_NUM_THREADS where the host
    sets it), then a shorter single-thread sample of the same rows.  `cores`
    is the thread count used; `host_cpus` gives nproc, the affinity mask and
    the thread limit it came from."""
    import oracle
    p = oracle.problem_of(inp)
    threads = oracle.default_threads()
    R = inp.w.B * inp.w.q_len * inp.w.Hq         # query rows of one step

    def timed_rows(rows, nthreads, budget):
        reps, t = 0, time.perf_counter()
        while True:
            oracle.attention(p, inp.q, inp.k, inp.v, seq_lens=inp.seq_lens, block_table=inp.block_table,
                             rows=rows, threads=nthreads)
            reps += 1
            el = time.perf_counter() - t
            if el >= budget or reps >= 1000:
                return reps, el

    # bounded sample: all rows when one step fits the budget, else a prefix of rows
    t = time.perf_counter()
    rows = np.arange(min(R, 8), dtype=np.int32)
    oracle.attention(p, inp.q, inp.k, inp.v, seq_lens=inp.seq_lens, block_table=inp.block_table, rows=rows,
                     threads=threads)
    per_row = (time.perf_counter() - t) / len(rows)
    n_rows = int(min(R, max(1, seconds / max(per_row, 1e-9))))
    rows = np.arange(n_rows, dtype=np.int32)
    reps, el = timed_rows(rows, threads, seconds)
    step_s = el / reps * (R / n_rows)          # scaled to a whole step
    n1 = max(1, min(n_rows, threads))          # single thread: a few of the same rows
    reps1, el1 = timed_rows(rows[:n1], 1, seconds / 4)
    step1_s = el1 / reps1 * (R / n1)
    return {"value": alg["step"] / step_s / 1e12, "unit": "TB/s", "cores": threads, "kind": "oracle",
            "host_cpus": oracle.host_cpus(),
            "us_per_step": step_s * 1e6, "single_thread_us_per_step": step1_s * 1e6, "cpu": _cpu_model(),
            "sample": f"{reps} x {n_rows}/{R} query rows of the same workload, {el:.1f} s of fp64 oracle work "
                      f"on {threads} threads, scaled to one step; single thread: {reps1} x {n1} rows, {el1:.1f} s"}


def run_settings(args):
    """The bench options that select which kernel runs and how."""
    s = {"kernel": args.kernel, "mode": args.mode}
    if args.merge != "separate":
        s["merge"] = args.merge
    if args.mode == "unified":
        s.update(phi=args.phi, lo=args.lo, hi=args.hi)
        if args.fallback != "split":
            s["fallback"] = args.fallback
    return s


def kernel_key(name):
    """Key of a kernel in the PMC summaries: the single-launch kernel, a
    split-partial kernel, the combine, or the name itself."""
    if "fused_mfma_kernel" in name:
        return "fused"
    if "partial" in name or "shared_kv" in name:
        return PARTIAL_KERNEL
    if "combine" in name:
        return "combine"
    return name[:60]


def traffic_from_profile(workload, kernel_keys, settings):
    """HBM bytes per timed call (the sum over `kernel_keys`, one launch each)
    from the committed PMC summary, if it was taken with the same kernel
    sources and run settings; else None.  kernel_keys may also be a list of
    such lists (the kernels a call may have launched): the first one the
    summary holds in full is used."""
    f = ROOT / "profiles" / f"{workload}_pmc.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    if d.get("source_hash") != source_hash() or d.get("settings") != settings:
        return None
    options = kernel_keys if kernel_keys and isinstance(kernel_keys[0], list) else [kernel_keys]
    kernels = d.get("kernels", {})
    for keys in options:
        if all(k in kernels for k in keys):
            return sum(kernels[k]["hbm_bytes_per_launch"] for k in keys)
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_gqa_32k")
    ap.add_argument("--mode", default="sync", choices=["sync", "unified"])
    ap.add_argument("--phi", type=float, default=-20.0)
    ap.add_argument("--lo", type=float, default=-20.0)
    ap.add_argument("--hi", type=float, default=20.0)
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--fallback", default="split", choices=["split", "row"],
                    help="unified max: recompute the flagged split, or every split of a flagged row")
    ap.add_argument("--merge", default=None, choices=["separate", "fused", "auto"],
                    help="separate: a contiguous cache through the partial and combine entry points (two "
                         "launches, timed one by one); fused / auto: fd_decode_attn (or the paged entry point) "
                         "with that merge mode.  Default: auto where it runs one kernel (a paged cache, one "
                         "split per row, the VALU kernel with at most 16 splits), else separate (what auto "
                         "picks there)")
    ap.add_argument("--split", type=int, default=0,
                    help="split size override (default: the workload's; a sweep knob, not the headline)")
    ap.add_argument("--warm", action="store_true", help="one KV copy (cache-resident for small caches)")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of one captured HIP graph instead of eager launches")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-profile", metavar="DIR")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a device-to-device copy of 256 MiB (a plain copy kernel of known size "
                         "for scaling HBM counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="combine rocprofv3 FETCH_SIZE and WRITE_SIZE runs into profiles/<workload>_pmc.json")
    args = ap.parse_args()
    if args.merge is None:
        args.merge = default_merge(args.workload, args.split, args.kernel)

    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return 0
    if args.pmc_summary:
        pmc_summary(args.workload, *args.pmc_summary, settings=run_settings(args))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the kernels run on the "
              f"KV share of a single MI355X; there is no multi-GPU path)", file=sys.stderr)
        return 2

    import synth
    w = synth.WORKLOADS[args.workload]
    if args.split:
        import dataclasses
        w = dataclasses.replace(w, split=args.split)
    log(f"[bench] generating {w.name}")
    inp = synth.make_inputs(w, poison_tail=False)
    alg = algorithmic_bytes(inp)
    g = run_gpu(args, inp, w)
    part_s = float(np.mean(g["part_us"])) * 1e-6
    step_s = g["step_ms"] * 1e-3
    parity = parity_spot_check(inp, g["res"], np.arange(0, w.B * w.q_len * w.Hq, max(1, (w.B * w.q_len * w.Hq) // 32)))
    log(f"[bench] step {g['step_ms'] * 1e3:.2f} us, partial {np.mean(g['part_us']):.2f} us, "
        f"combine {np.mean(g['comb_us']):.2f} us (back-to-back averages); parity {parity}")
    kname = "fd_decode_attn_paged" if w.page_size else ("fd_decode_attn" if args.merge != "separate" else PARTIAL_KERNEL)
    # the kernels one timed call launches: the entry points with a merge run the
    # partial and the combine, or the single fused kernel
    if kname == PARTIAL_KERNEL:
        keys = [PARTIAL_KERNEL]
    elif args.merge == "fused":
        keys = ["fused"]
    elif args.merge == "separate":
        keys = [PARTIAL_KERNEL, "combine"]
    else:   # auto: whichever the library took (the partial kernel alone: one split, direct output)
        keys = [["fused"], [PARTIAL_KERNEL, "combine"], [PARTIAL_KERNEL]]
    traffic = traffic_from_profile(w.name, keys, run_settings(args))
    bound, peak = roofline_bound(w, args.kernel, alg)
    if bound == "hbm":
        achieved, unit = alg["partial"] / part_s / 1e9, "GB/s"
    else:
        achieved, unit = alg["flops"] / part_s / 1e12, "TFLOP/s"
    line = {
        "metric": "decode-attn us/step and achieved HBM TB/s (% of MI355X peak), N=32k GQA",
        "value": alg["step"] / step_s / 1e12,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": g["steps"],
        "warmup": args.warmup,
        "ms_per_step": g["step_ms"],
        "us_per_step": g["step_ms"] * 1e3,
        "pct_of_hbm_peak": 100.0 * alg["step"] / step_s / 1e9 / HBM_PEAK_GBPS,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "N": w.N, "q_len": w.q_len,
                   "kv_dtype": w.dtype, "split": w.split, "num_splits": g["S"], "page_size": w.page_size,
                   "softmax": args.mode, "kernel": args.kernel, "merge": args.merge, "kv_copies": g["copies"],
                   "launch": "hip graph" if args.graph else "eager",
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single GPU"},
        "kernels_us": {"partial": float(np.mean(g["part_us"])), "combine": float(np.mean(g["comb_us"])),
                       "timing": "HIP events around K back-to-back launches of each kernel"},
        "roofline": {"bound": bound, "kernel": kname, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg["partial"], "per_unit_bytes": alg["per_unit"],
                     "units_per_launch": alg["units"], "algorithmic_flops_per_launch": alg["flops"],
                     "hbm_gbps": alg["partial"] / part_s / 1e9, "tflops": alg["flops"] / part_s / 1e12},
        "parity": parity,
        "device": g["device"],
    }
    if args.mode == "unified":
        line["fallback"] = fallback_stats(inp, g["res"]["flags"], args)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(inp, alg, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0 if parity["ok"] else 1


# ----------------------------------------------------------------------------
# rocprofv3 output -> markdown
# ----------------------------------------------------------------------------
def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_profile(d):
    d = Path(d)
    for f in sorted(glob.glob(str(d / "**" / "*kernel_stats.csv"), recursive=True)):
        rows = _read_csv(f)
        print(f"### kernel stats ({Path(f).name})\n")
        print("| kernel | calls | avg (us) | min (us) | max (us) | total % |")
        print("|---|---|---|---|---|---|")
        for r in rows:
            name = r.get("Name", "")
            short = name if len(name) < 90 else name[:87] + "..."
            print(f"| `{short}` | {r.get('Calls')} | {float(r.get('AverageNs', 0)) / 1e3:.2f} | "
                  f"{float(r.get('MinNs', 0)) / 1e3:.2f} | {float(r.get('MaxNs', 0)) / 1e3:.2f} | "
                  f"{float(r.get('Percentage', 0)):.1f} |")
        print()
    for f in sorted(glob.glob(str(d / "**" / "*counter_collection.csv"), recursive=True)):
        rows = _read_csv(f)
        agg = {}
        for r in rows:
            key = (r.get("Kernel_Name", ""), r.get("Counter_Name", ""))
            agg.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
        print(f"### counters ({Path(f).name})\n")
        print("| kernel | counter | dispatches | mean per dispatch |")
        print("|---|---|---|---|")
        for (kn, cn), vals in sorted(agg.items()):
            short = kn if len(kn) < 90 else kn[:87] + "..."
            print(f"| `{short}` | {cn} | {len(vals)} | {np.mean(vals):.1f} |")
        print()


def _counter_rows(d, counter):
    rows = []
    for f in glob.glob(str(Path(d) / "**" / "*counter_collection.csv"), recursive=True):
        rows += [r for r in _read_csv(f) if r.get("Counter_Name") == counter]
    rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
    return rows


def _counter_means(d, counter):
    """{kernel name: (dispatches, mean counter value per dispatch)} of one --pmc
    run; the calibration copy is keyed "calibration copy" (the first three
    copy dispatches, issued before any input upload)."""
    agg = {}
    copies = 0
    for r in _counter_rows(d, counter):
        name = r.get("Kernel_Name", "")
        if "copyBuffer" in name:
            if copies >= 3:
                continue
            copies += 1
            name = "calibration copy"
        agg.setdefault(name, []).append(float(r.get("Counter_Value", 0)))
    return {k: (len(v), float(np.mean(v))) for k, v in agg.items()}


def pmc_summary(workload, fetch_dir, write_dir, settings):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the calibration copy of
    COPY_BYTES.  Writes profiles/<workload>_pmc.json and prints a table.
    settings: the run options the counter runs used (pass the same ones)."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    copy_name = "calibration copy" if "calibration copy" in fetch else None
    if copy_name is None:
        raise SystemExit("no calibration copy kernel in the FETCH_SIZE run (use --copy-calibration)")
    f_scale = COPY_BYTES / (fetch[copy_name][1] * 1024)
    w_scale = COPY_BYTES / (write[copy_name][1] * 1024)
    out = {"workload": workload, "source_hash": source_hash(), "settings": settings, "copy_bytes": COPY_BYTES,
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    print(f"| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/launch (scaled) |")
    print("|---|---|---|---|---|")
    for name in sorted(set(fetch) | set(write)):
        fk = fetch.get(name, (0, 0.0))
        wk = write.get(name, (0, 0.0))
        hbm = fk[1] * 1024 * f_scale + wk[1] * 1024 * w_scale
        key = kernel_key(name)
        out["kernels"][key] = {"name": name, "fetch_kib": fk[1], "write_kib": wk[1], "hbm_bytes_per_launch": hbm,
                               "dispatches": max(fk[0], wk[0])}
        short = name if len(name) < 80 else name[:77] + "..."
        print(f"| `{short}` | {max(fk[0], wk[0])} | {fk[1]:.1f} | {wk[1]:.1f} | {hbm:.4g} |")
    print(f"\ncalibration: copy of {COPY_BYTES} B read as FETCH_SIZE x{f_scale:.4f}, WRITE_SIZE x{w_scale:.4f}")
    (ROOT / "profiles").mkdir(exist_ok=True)
    (ROOT / "profiles" / f"{workload}_pmc.json").write_text(json.dumps(out, indent=1) + "\n")


if __name__ == "__main__":
    sys.exit(main())
