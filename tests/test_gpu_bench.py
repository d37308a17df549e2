"""The benchmark's output contract on a short run: one JSON line with the
headline metric, the roofline of the dominant kernel and the per-row figures
(the CPU baseline is skipped here; its timing loop is plain host code)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_keys():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = subprocess.run([sys.executable, "bench.py", "--steps", "5", "--warmup", "5", "--no-cpu"], cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 5 and d["value"] > 0
    assert d["config"]["workload"] == "dit_attn_proj_2640x3072x3072"
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert d["settle_ms"] > 0
    for row in ("tiny_linear", "kv_quant", "kv_quant_4over6", "kv_dequant", "kv_window_attention",
                "rht16_quantize", "wgrad_gemm", "ffn_pair", "train_linear_triple"):
        assert d["rows"][row]["ms"] > 0, row
    assert d["rows"]["tiny_linear"]["us"] > 0


@pytest.mark.gpu
def test_bench_runs_one_named_row_alone():
    """--only / --no-headline (used for profiling one shape per kernel): only
    the named row is measured and the headline keys are absent."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = subprocess.run([sys.executable, "bench.py", "--steps", "5", "--warmup", "2", "--no-cpu", "--no-headline",
                        "--only", "tiny_linear"], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert "value" not in d and list(d["rows"]) == ["tiny_linear"]


def test_bench_refuses_more_than_one_gpu():
    """CPU-only: the argument check runs before anything touches a GPU."""
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
    r = subprocess.run([sys.executable, "bench.py", "--only", "no_such_row"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "unknown rows" in r.stderr
