"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
algorithmic byte counts the roofline divides by, and the HBM-counter scaling
that turns rocprofv3's FETCH_SIZE / WRITE_SIZE into bytes per launch."""
import csv
import json
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest

import bench
import synth

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def test_algorithmic_bytes_of_the_headline_shape():
    # B=1, Hq=32, Hkv=8, d=128, N=32768, bf16: K and V of every (KV head, token)
    # once, 2 * 128 * 2 = 512 bytes per unit, plus q (and out for the step)
    inp = synth.make_inputs(synth.WORKLOADS["long_gqa_32k"], poison_tail=False)
    a = bench.algorithmic_bytes(inp)
    assert a["per_unit"] == 512 and a["units"] == 32768 * 8
    assert a["kv"] == 32768 * 8 * 512
    assert a["q"] == a["out"] == 32 * 128 * 2
    assert a["partial"] == 134_225_920 and a["step"] == 134_225_920 + 8192 and a["table"] == 0


def test_algorithmic_bytes_count_the_block_table_entries_read():
    w = synth.with_lens(synth.Workload("t", B=3, Hq=8, Hkv=2, d=64, dtype="f16", split=64, N=1, page_size=16),
                        (17, 16, 1000))
    inp = synth.make_inputs(w, poison_tail=False)
    a = bench.algorithmic_bytes(inp)
    pages = 2 + 1 + 63
    assert a["table"] == 4 * pages
    assert a["kv"] == (17 + 16 + 1000) * 2 * 2 * 64 * 2
    assert a["units"] == (17 + 16 + 1000) * 2


def test_flops_and_bound_decode_and_prefill():
    # decode: 4 d flops per (query row, token): 32 heads x 32768 tokens; HBM-bound
    inp = synth.make_inputs(synth.WORKLOADS["long_gqa_32k"], poison_tail=False)
    a = bench.algorithmic_bytes(inp)
    assert a["flops"] == 4 * 128 * 32 * 32768
    assert bench.roofline_bound(inp.w, "auto", a) == ("hbm", bench.HBM_PEAK_GBPS)
    # a whole 4k prompt: token i sees i + 1 tokens, sum N (N + 1) / 2; matrix-bound
    w = synth.WORKLOADS["prefill_gqa_4k"]
    inp = synth.make_inputs(w, poison_tail=False)
    a = bench.algorithmic_bytes(inp)
    assert a["flops"] == 4 * 128 * 32 * (4096 * 4097 // 2)
    assert bench.roofline_bound(w, "auto", a) == ("mfma", bench.MFMA_PEAK_TFLOPS)
    # chunk of the last 3 of 5 tokens and a request shorter than its queries
    w = synth.with_lens(synth.Workload("c", B=2, Hq=2, Hkv=1, d=8, dtype="f32", split=8, N=1, q_len=3), (5, 2))
    a = bench.algorithmic_bytes(synth.make_inputs(w, poison_tail=False))
    assert a["flops"] == 4 * 8 * 2 * ((3 + 4 + 5) + (0 + 1 + 2))


def _write_counters(d: Path, counter, rows):
    d.mkdir(parents=True)
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_bytes_are_scaled_by_the_calibration_copy(tmp_path, monkeypatch):
    """A copy of COPY_BYTES reads as FETCH_SIZE = half its bytes and WRITE_SIZE
    = all of them (the factors measured on MI355X); a kernel's counters scale by
    the same factors, and only the first three copy dispatches calibrate."""
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    monkeypatch.setattr(bench, "source_hash", lambda: "h")
    kib = bench.COPY_BYTES / 1024
    partial = "void fd::partial_mfma_kernel<2, 128, 4, 1, false, false>(fd::PartialParams)"
    copy = "__amd_rocclr_copyBuffer"
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(copy, kib / 2)] * 3 + [(copy, 5.0), (partial, 1000.0),
                                                                           (partial, 1002.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(copy, kib)] * 3 + [(copy, 7.0), (partial, 10.0), (partial, 10.0)])
    settings = {"kernel": "auto", "mode": "sync"}
    bench.pmc_summary("wl", tmp_path / "f", tmp_path / "w", settings)
    d = json.loads((tmp_path / "profiles" / "wl_pmc.json").read_text())
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    expect = 1001.0 * 1024 * 2.0 + 10.0 * 1024 * 1.0
    assert d["kernels"][bench.PARTIAL_KERNEL]["hbm_bytes_per_launch"] == pytest.approx(expect)
    assert bench.traffic_from_profile("wl", [bench.PARTIAL_KERNEL], settings) == pytest.approx(expect)
    # a call of two kernels sums them; a kernel without counters gives none
    assert bench.traffic_from_profile("wl", [bench.PARTIAL_KERNEL, bench.PARTIAL_KERNEL], settings) == \
        pytest.approx(2 * expect)
    assert bench.traffic_from_profile("wl", [bench.PARTIAL_KERNEL, "combine"], settings) is None
    # other settings, or other kernel sources, make the stored figure stale
    assert bench.traffic_from_profile("wl", [bench.PARTIAL_KERNEL], {"kernel": "valu", "mode": "sync"}) is None
    monkeypatch.setattr(bench, "source_hash", lambda: "changed")
    assert bench.traffic_from_profile("wl", [bench.PARTIAL_KERNEL], settings) is None


def test_kernel_keys():
    assert bench.kernel_key("void fd::(anonymous namespace)::fused_mfma_kernel<2, 128, 4, 4, false, false>"
                            "(fd::PartialParams)") == "fused"
    assert bench.kernel_key("void fd::(anonymous namespace)::partial_valu_kernel<2, 128, 4, false, true>"
                            "(fd::PartialParams)") == bench.PARTIAL_KERNEL
    assert bench.kernel_key("void fd::(anonymous namespace)::combine_kernel<128, 128, 256, true>"
                            "(fd::CombineParams)") == "combine"
    assert bench.kernel_key("void fd::(anonymous namespace)::shared_kv_mfma_kernel<2, 128, false, true>"
                            "(fd::PartialParams)") == bench.PARTIAL_KERNEL


def test_default_merge_follows_the_library_auto_choice():
    """Two launches timed apart where AUTO merges separately; one call where
    AUTO runs a single kernel (paged cache, one split per row, the VALU
    kernel with at most 16 splits)."""
    assert bench.default_merge("long_gqa_32k") == "separate"
    assert bench.default_merge("llama2_7b_mha") == "separate"
    assert bench.default_merge("llama2_7b_mha", kernel="valu") == "auto"       # 16 splits
    assert bench.default_merge("long_gqa_32k", kernel="valu") == "separate"    # 128 splits
    assert bench.default_merge("tiny_mha") == "auto"                           # fp32: VALU, 4 splits
    assert bench.default_merge("prefill_gqa_4k") == "auto"                     # one split per row
    assert bench.default_merge("paged_batched_gqa") == "auto"
    assert bench.default_merge("long_gqa_32k", split=32768) == "auto"
