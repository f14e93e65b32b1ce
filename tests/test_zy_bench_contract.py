"""bench.py's command-line contract: one GPU only, and one JSON line with the fields the
benchmark record needs (metric, value, unit, step counts, the roofline of the dominant kernel and
the CPU-oracle baseline)."""
from __future__ import annotations

import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused(capsys):
    import bench
    assert bench.main(["--gpus", "2"]) == 2
    err = capsys.readouterr().err
    assert "one GPU" in err


@pytest.mark.gpu
def test_bench_json_line(capsys):
    import bench
    rc = bench.main(["--workload", "tiny_b1_h4_d64_t256_f32", "--steps", "3", "--warmup", "1",
                     "--no-copy-ceiling", "--cpu-budget", "0.5"])
    assert rc in (None, 0)
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["config"]["workload"] == "tiny_b1_h4_d64_t256_f32"
    # decode tokens/s is the batch over the step time
    assert rec["value"] == pytest.approx(rec["config"]["batch"] / (rec["ms_per_step"] * 1e-3), rel=1e-6)
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    base = rec["cpu_baseline"]
    assert base["kind"] == "oracle" and base["value"] > 0 and base["cores"] >= 1
