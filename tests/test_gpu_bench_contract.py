"""The bench's one-line JSON report: a short run of the default workload and
of a multi-token one, checked for the fields and units the report promises."""
import json
import os
import subprocess
import sys

import pytest

from gpu_common import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", *args], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, p.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("config", [None, "verify"])
def test_report_fields(config):
    say(f"case: bench report, config {config or 'default'}")
    d = _bench(*(["--config", config] if config else []))
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0 and isinstance(d["config"]["workload"], str)
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    if config is None:
        # the default: the agentic workload with the shared-prefix (cascade)
        # decode, the per-sequence decode timed beside it
        assert d["unit"] == "GB/s" and d["config"]["workload"].startswith("agentic")
        assert "cascade decode" in d["config"]["workload"]
        assert d["plain_decode_us"] > 0 and d["plain_value"] > 0
        # the measured ceilings of the same GPU and where the kernels stand
        c = d["ceilings"]
        assert "error" not in c, c
        for k in ("stream_read_GBps", "record_gather_GBps", "mixed_7r2w_GBps", "mixed_7r2w_scattered_GBps"):
            assert 0 < c[k] < c["peak_GBps"], k
        assert 0 < c["quantize_frac_of_mixed_scattered"] < 1.5
        assert 0 < c["decode_unique_frac_of_record_gather"] < 1.5
