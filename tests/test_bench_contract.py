"""bench.py's output contract: one JSON line with the fields a benchmark
driver reads, one GPU only, and the source hash that keys the committed
traffic counters (comments and layout do not count, code does)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one" in r.stderr and r.stdout == ""


def test_source_hash_ignores_comments_and_layout():
    a = "int f(int x) {\n  return x + 1;  // one\n}\n"
    b = "/* header */\nint f(int x)\n{ return x + 1; }\n"
    c = "int f(int x) { return x + 2; }\n"
    assert bench.code_text(a) == bench.code_text(b) != bench.code_text(c)
    files = {p: open(os.path.join(ROOT, p), encoding="utf-8").read() for p in bench.FWD_KERNEL_SOURCES}
    base = bench.kernel_source_hash(lambda p: files[p])
    first = bench.FWD_KERNEL_SOURCES[0]
    assert bench.kernel_source_hash(lambda p: files[p] + "\n// a note\n") == base
    assert bench.kernel_source_hash(lambda p: files[p] + ("\nstatic int extra;\n" if p == first else "")) != base


def test_algorithmic_bytes_of_the_70b_shard():
    import workloads as W
    w = W.BY_NAME["shard70b"]
    assert bench.fwd_bytes(w, 2048) == 369_164_288
    assert bench.bwd_bytes(w, 2048) == 100_761_600


@pytest.mark.gpu
def test_bench_prints_one_contract_line(cuda_device):
    print("[bench-contract] tiny, 3 steps", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline", "--no-extras"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0 and rec["higher_is_better"] is True
    assert rec["unit"] == "tokens/s" and rec["dtype"] == "f32" and rec["config"]["workload"] == "tiny"
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-12
    assert rec["cpu_baseline"] is None and rec["extras"] is None
    # The other workloads of the configuration list, each with its own step,
    # kernel times and fractions of peak.
    cfg = rec["configs"]
    assert sorted(cfg) == ["c1", "c2", "c4", "c5"]
    names = {"c1": "tiny", "c2": "page_demo", "c4": "ragged13b", "c5": "long128k"}
    for tag, c in cfg.items():
        assert c["workload"] == names[tag] and c["local_tokens"] > 0
        for key in ("step_us_wall", "step_us_graph_replay", "fwd_us", "bwd_us", "tokens_per_s_wall",
                    "tokens_per_s_kernels", "fwd_bwd_pct_of_peak", "fwd_frac"):
            assert c[key] > 0, (tag, key)
        assert abs(c["tokens_per_s_kernels"] - c["local_tokens"] / ((c["fwd_us"] + c["bwd_us"]) * 1e-6)) < 1e-6 * c[
            "tokens_per_s_kernels"]
        assert "cpu_baseline" not in c
