"""Host-side checks of the benchmark (no GPU): the one-GPU contract and the rule that a
committed traffic figure is used only for the kernel sources it was taken on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_figure_follows_the_kernel_sources(monkeypatch):
    wl = "llama3_8b_decode_bf16_B16_H32_G8_d128_n4096"
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl}.json")) as f:
        t = json.load(f)
    assert t["kernel"] == "decode_mfma_kernel"
    # each counter is scaled by its own reading for a copy of known size
    cal = t["copy_calibration"]
    assert abs(cal["fetch_factor"] - cal["bytes"] / 1024 / cal["fetch_size_kib"]) < 1e-3
    assert abs(cal["write_factor"] - cal["bytes"] / 1024 / cal["write_size_kib"]) < 1e-3
    want = t["hbm_bytes_per_launch"] if t["kernel_source_sha"] == bench.kernel_source_hash() else None
    assert bench.load_traffic(wl) == want
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic(wl) is None
    assert bench.load_traffic("no_such_workload") is None


def test_kernel_source_hash_covers_the_decode_sources():
    assert set(bench.KERNEL_SOURCES) == {"decode_mfma.hip", "decode_valu.hip", "gqa_internal.h", "mfma_common.h"}
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_source_hash()


def test_per_config_entry_reads_a_child_line():
    import bench
    line = {"ms_per_step": 0.1105, "value": 4860.0, "pct_of_hbm_peak": 60.75, "tokens_per_s": 289592.8,
            "kernel_ms": {"split_decode": 0.1012, "lse_merge": 0.0083},
            "roofline": {"frac": 0.6633, "bound": "hbm", "traffic": None}}
    e = bench.per_config_entry(line)
    assert e == {"step_us": 110.5, "kv_gbps": 4860.0, "pct_of_hbm_peak": 60.75, "tokens_per_s": 289592.8,
                 "decode_us": 101.2, "merge_us": 8.3, "decode_roofline_frac": 0.6633, "roofline_bound": "hbm",
                 "traffic": None}


def test_decode_kernel_name_follows_the_plan():
    # a group split into row blocks runs the re-reading form of the matrix-core kernel
    assert bench.decode_kernel_name({"policy": "mfma", "row_blocks": 1}) == "decode_mfma_kernel"
    assert bench.decode_kernel_name({"policy": "mfma", "row_blocks": 4}) == "decode_mfma_reread_kernel"
    assert bench.decode_kernel_name({"policy": "valu", "row_blocks": 1}) == "decode_valu_kernel"
