"""The benchmark's JSON line on a real GPU: one short run of `bench.py` on the smallest
bf16 long-context-shaped configuration, in a process of its own, checked against the
line's contract (metric and unit, one GPU, exact step counts, the roofline object for
the decode kernel and the CPU baseline object)."""
import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bench_line_contract():
    wl = "llama3_8b_decode_bf16_B16_H32_G8_d128_n4096"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", wl, "--steps", "7",
                        "--warmup", "2", "--no-ceiling", "--cpu-budget", "1"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.strip().splitlines() if x.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["n_gpus"] == 1
    assert d["steps"] == 7 and d["warmup"] == 2 and d["scaling"] == "weak" and d["dtype"] == "bf16"
    assert d["config"]["workload"] == wl and d["vs_baseline"] is None
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # KV GB/s from the workload's bytes and the step time
    assert abs(d["value"] - d["config"]["kv_bytes"] / (d["ms_per_step"] * 1e-3) / 1e9) < 1e-2 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert rf["peak"] == (8000.0 if rf["bound"] == "hbm" else 2500.0)
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0.0 < rf["frac"] < 1.0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert d["per_config"] is None   # only the default run measures the other configurations
