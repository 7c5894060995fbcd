"""bench.py's output contract: one JSON line with the keys the driver reads.

The GPU case runs one short in-process bench of the tiny workload (so the
line's shape is checked on the same code path the driver runs); the CPU case
checks that a multi-GPU request is refused with an explanation."""
import io
import json
import os
import sys
from contextlib import redirect_stdout

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

REQUIRED = {"metric": str, "value": float, "unit": str, "n_gpus": int, "steps": int,
            "warmup": int, "ms_per_step": float, "higher_is_better": bool, "scaling": str,
            "dtype": str, "data": str, "config": dict, "roofline": dict}


def _line(argv):
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.main(argv)
    lines = [l for l in buf.getvalue().splitlines() if l.startswith("{")]
    assert len(lines) == 1, buf.getvalue()
    return json.loads(lines[0])


def test_more_than_one_gpu_is_refused():
    buf = io.StringIO()
    with redirect_stdout(buf), pytest.raises(SystemExit) as ei:
        bench.main(["--gpus", "2"])
    assert ei.value.code == 2
    msg = json.loads(buf.getvalue().strip())
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


@pytest.mark.gpu
def test_bench_line_carries_the_contract_keys():
    d = _line(["--only", "--config", "tiny", "--steps", "2", "--warmup", "1",
               "--precondition-s", "0", "--cpu-seconds", "0.2"])
    for k, t in REQUIRED.items():
        assert isinstance(d[k], t), (k, d.get(k))
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"].startswith("tiny")
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == d["unit"] and c["value"] > 0
    assert c["cores"] >= 1 and c["sample"]
    assert set(d["arms"]) == {"planned", "call", "fixed", "graph"}
