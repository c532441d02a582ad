"""bench.py on the GPU: a short run prints one JSON line with the fields the
benchmark contract asks for (throughput, its roofline against the published
peak, the decode roofline, the CPU baseline)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    print("case: bench.py --steps 2 --warmup 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1"], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert roof["achieved"] == d["value"]
    dec = d["decode"]["roofline"]
    assert dec["bound"] == "hbm" and dec["unit"] == "GB/s" and dec["peak"] == 8000.0
    assert 0 < dec["frac"] < 1
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["blas"]
    # the N = 16384 prefill is timed in the same step, with its own roofline
    # and an oracle baseline on sampled rows
    lp = d["long_prefill"]
    assert lp["value"] > 0 and lp["roofline"]["peak"] == 2500.0
    assert abs(lp["roofline"]["frac"] - lp["value"] / 2500.0) < 1e-9
    assert lp["cpu_baseline"]["kind"] == "oracle" and lp["cpu_baseline"]["value"] > 0
    ach = d["achievable"]
    assert ach["mfma_bf16_TFLOPs"] > 0 and ach["random_4k_read_GBps"] > 0
    assert 0 < roof["frac_of_achievable"] and 0 < dec["frac_of_achievable"]
    sd = d["shared_decode"]
    assert sd["cold"]["shared_ms"] > 0 and sd["warm"]["shared_ms"] > 0
