"""bench.py: its one-line JSON contract and the host logic behind the figures.

CPU tests cover:
- the refusal of more than one GPU;
- the algorithmic-bytes formulas of the step and the embedding layer;
- the guards on the committed traffic file;
- the CPU-baseline record.

The GPU test runs a short bench and checks every key of its JSON line.
"""

import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_algorithmic_bytes():
    # fp32 params, bf16 grads: read p 4, g 2, two codes 2; write p 4, two codes 2; both
    # block maxima read and written (16 B per block)
    assert bench.algorithmic_bytes([2048], 4, 2) == 2048 * 14 + 16
    assert bench.algorithmic_bytes([2049], 4, 2) == 2049 * 14 + 2 * 16
    assert bench.algorithmic_bytes([1, 2048], 2, 2) == 1 * 10 + 16 + 2048 * 10 + 16
    assert bench.algorithmic_bytes([2048], 4, 4) == 2048 * 16 + 16
    assert bench.algorithmic_bytes([], 4, 2) == 0


def test_embedding_bytes():
    # forward: 3 distinct fp32 rows of 8, 5 bf16 output rows, 16 B per token, gamma and beta
    fwd, bwd = bench.embedding_bytes(3, 5, 8)
    assert fwd == 3 * 32 + 5 * 16 + 5 * 16 + 2 * 32
    # backward: the same reads, each distinct row's fp32 gradient read and written, gamma
    # read, dgamma and dbeta written; nothing for the workspace
    assert bwd == 3 * 32 + 5 * 16 + 5 * 16 + 3 * 64 + 3 * 32
    # the embedding workload's figures: 12,999 distinct rows of 4096, 65,536 tokens
    assert bench.embedding_bytes(12999, 65536, 4096)[1] == 1_176_895_488


def test_kernel_code_hash_ignores_comments_only():
    src = open(bench.KERNEL_SRC).read()
    h = bench.kernel_code_hash()
    assert h == bench.kernel_code_hash(src)
    assert bench.kernel_code_hash("// a note\n" + src.replace("\n", "\n  ") + "\n/* more */") == h
    # a changed constant in the code is a changed kernel
    assert bench.kernel_code_hash(src.replace("0x1p-19f", "0x1p-20f")) != h
    assert bench.kernel_code_hash(src.replace("kStepRun = 2", "kStepRun = 4")) != h


def test_traffic_file_guards(tmp_path, monkeypatch):
    sha = bench.kernel_code_hash()
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.load_traffic("llama7b") is None                      # no file
    path.write_text("not json")
    assert bench.load_traffic("llama7b") is None
    good = {"workload": "llama7b", "kernel_code_sha256": sha, "traffic_bytes_per_launch": 123}
    path.write_text(json.dumps(good))
    assert bench.load_traffic("llama7b") == 123
    assert bench.load_traffic("gpt1p3b") is None                      # other workload
    path.write_text(json.dumps(dict(good, kernel_code_sha256="0" * 64)))
    assert bench.load_traffic("llama7b") is None                      # kernel changed since


def test_cpu_baseline_record():
    r = bench.cpu_baseline(target_seconds=0.1)
    assert set(r) == {"value", "unit", "cores", "kind", "sample"}
    assert r["kind"] == "oracle" and r["unit"] == "params/s" and r["cores"] == 1
    assert r["value"] > 0 and "4,194,304 params" in r["sample"]


@pytest.mark.gpu
@pytest.mark.parametrize("layout", ["flat", "params"])
def test_bench_json_line(layout):
    """A short run on the GPT-1.3B set prints exactly one JSON line with the contract's
    keys, and its roofline figures are consistent with each other."""
    print(f"bench gpt1p3b layout {layout}", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload",
                        "gpt1p3b", "--layout", layout, "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["metric"] == bench.METRIC and d["unit"] == "params/s"
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["dtype"] == "f32" and d["data"] == "synthetic" and d["cpu_baseline"] is None
    c = d["config"]
    assert c["workload"].startswith("gpt1p3b") and c["layout"] == layout
    assert c["params"] == 1_311_086_592 and c["tensors"] == 243
    assert d["value"] == pytest.approx(c["params"] / (d["ms_per_step"] * 1e-3), rel=1e-3)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert rf["traffic"] is None                     # counters were taken on llama7b
    launch_bytes = c["algorithmic_bytes_per_step"] / rf["launches_per_step"]
    assert rf["algorithmic_bytes_per_launch"] == int(launch_bytes)
    assert rf["achieved"] == pytest.approx(launch_bytes / (rf["avg_launch_ms"] * 1e-3) / 1e9,
                                           rel=2e-3)
    assert 1000 < rf["achieved"] < 8000
