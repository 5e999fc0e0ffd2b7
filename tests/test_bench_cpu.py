"""CPU tests of bench.py's own contract: the one-GPU guard, the HBM traffic
summary built from two rocprofv3 counter runs (calibration against the
ring-receive copies, the per-dispatch sum), the source-hash gate that nulls a
stale summary, and the CPU-baseline record (the oracle timed on a sample).
No GPU is used."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


@pytest.mark.parametrize("which", ["bf16", "fp8"])
def test_traffic_summary_scales_by_the_copy_kernels(tmp_path, which):
    k = bench.KERNELS[which]
    blk_kib = k["copy_bytes"] / 1024
    attn = f"void cpattn::(anonymous namespace)::{k['name']}(cpattn::BlockArgs)"
    # the copies read back half of what they move through FETCH_SIZE (factor 2) and all of it through WRITE_SIZE
    fetch = [(bench.COPY_KERNEL, blk_kib / 2), (attn, 1000.0), (bench.COPY_KERNEL, blk_kib / 2), (attn, 3000.0),
             (bench.COPY_KERNEL, 4.0)]                       # a small upload copy, outside the calibration band
    write = [(bench.COPY_KERNEL, blk_kib), (attn, 500.0), (bench.COPY_KERNEL, blk_kib), (attn, 700.0)]
    _counter_csv(tmp_path / "F", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "W", "WRITE_SIZE", write)
    out = tmp_path / "t.json"
    res = bench.summarize_pmc(str(tmp_path / "F"), str(tmp_path / "W"), which, out=str(out))
    assert res["fetch"]["factor"] == pytest.approx(2.0) and res["write"]["factor"] == pytest.approx(1.0)
    assert res["traffic_bytes_per_dispatch"] == pytest.approx([(2 * 1000 + 500) * 1024, (2 * 3000 + 700) * 1024])
    assert res["kernel"] == k["name"] and res["kernel_source_sha256"] == bench.kernel_sha256(which)
    assert json.loads(out.read_text()) == json.loads(json.dumps(res))


def test_stale_traffic_summary_is_not_reported(tmp_path, monkeypatch):
    profiles = tmp_path / "profiles"
    profiles.mkdir()
    good = {"kernel_source_sha256": bench.kernel_sha256("bf16"), "traffic_bytes_mean": 123.0}
    (profiles / bench.KERNELS["bf16"]["json"]).write_text(json.dumps(good))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the hash covers the real sources (the ROOT swap only redirects the summary file)
    monkeypatch.setattr(bench, "kernel_sha256", lambda which="bf16": good["kernel_source_sha256"])
    assert bench.measured_traffic("bf16") == 123.0
    monkeypatch.setattr(bench, "kernel_sha256", lambda which="bf16": "0" * 64)
    assert bench.measured_traffic("bf16") is None
    assert bench.measured_traffic("fp8") is None                   # no summary file at all


def test_committed_traffic_summaries_match_the_sources():
    for which in bench.KERNELS:
        t = bench.measured_traffic(which)
        assert t is not None and t > 0, f"{which}: committed traffic summary missing or stale"


def test_cpu_baseline_record():
    from harness.inputs import ShardSpec, make_inputs
    spec = ShardSpec(S=512, N=4, H=2, d=64, dtype="f32", mask="causal", rank=3, cfg_id=7)
    inp = make_inputs(spec, seed=0)
    r = bench.cpu_baseline(spec, inp["q"][3], inp["k"], inp["v"], 16)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0 and r["cores"] >= 1
    rows = np.linspace(0, spec.L - 1, 16).astype(np.int64)
    assert f"({int(np.sum(3 * spec.L + rows + 1))} visible pairs" in r["sample"]
    assert "of 2 (" in r["sample"]
