"""bench.py on the GPU (needs an MI355X): one short run of the 4-row
next-token workload in a subprocess prints one JSON line with the fields the
benchmark contract names, a roofline against the 8 TB/s HBM peak, the
lp_compute_ragged and probe legs, and no parity mismatch on the rows it
recomputes with the oracle."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_on_a_small_workload():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, "bench.py", "--workload", "no_echo_next_token",
                        "--no-decode", "--steps", "20", "--warmup", "20"],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 20
    assert d["config"]["workload"] == "no_echo_next_token"
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert d["value"] == pytest.approx(d["config"]["read_rows"] / (d["ms_per_step"] * 1e-3))
    assert d["compute_ragged"]["median_us"] > 0 and d["probe"]["us"] > 0
    assert d["compute_noalloc"]["median_us"] > 0
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["value"] > 0
    checks = d["cpu_baseline"]["timed_rows_check"]
    assert checks and all(c["mismatches"] == 0 and c["rows_checked"] > 0 for c in checks)
