"""bench.py keeps its output contract: one JSON line with the required fields
(GPU), and a clear refusal of more than one GPU (CPU)."""
import contextlib
import io
import json
import sys

import pytest

import bench


def _run(argv):
    out = io.StringIO()
    old = sys.argv
    sys.argv = ["bench.py"] + argv
    try:
        with contextlib.redirect_stdout(out):
            rc = bench.main()
    finally:
        sys.argv = old
    return rc, out.getvalue()


def test_more_than_one_gpu_is_refused(capsys):
    rc, out = _run(["--gpus", "2"])
    assert rc == 2 and out == ""
    assert "single-GPU" in capsys.readouterr().err


@pytest.mark.gpu
def test_json_line_fields():
    rc, out = _run(["--config", "1", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.2"])
    assert rc == 0
    lines = [l for l in out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert d["higher_is_better"] is True and d["data"] == "synthetic" and "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # the default (pipelined) schedule runs the dedup on a second stream: the
    # roofline kernel is a main-stream one
    assert d["schedule"] == "pipeline"
    assert r["kernel"] not in ("keys", "sort_hist", "sort_scan", "sort_scatter", "rle")
    assert "traffic" in r and "l2_hit_rate" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] == 1 and c["value"] > 0 and c["unit"] == d["unit"]
    # the oracle timed per phase, with the GPU's byte formula
    for ph in ("fwd", "bwd_update"):
        assert c[ph]["lookups_per_s"] > 0 and c[ph]["alg_GBps"] > 0 and c[ph]["s"] > 0
    assert "per_config" not in d          # only the headline workload carries the other configs


@pytest.mark.gpu
def test_pipeline_two_ahead_runs():
    rc, out = _run(["--config", "2", "--steps", "4", "--warmup", "2", "--ahead", "2", "--no-cpu-baseline",
                    "--single-schedule"])
    assert rc == 0
    d = json.loads([l for l in out.splitlines() if l.startswith("{")][0])
    assert d["schedule"].startswith("pipeline") and d["value"] > 0
