"""The benchmark's output contract: host-side pieces on the CPU, one short timed run on the GPU.

The GPU case runs bench.main in this process (a few steps of the headline workload, no CPU baseline
and no ceiling probes) and checks the one JSON line it prints: the fields a reader relies on and
the arithmetic that ties them together (value from the visible pairs and the step time, the
roofline fraction from its achieved and peak figures).
"""
import json
import os
import subprocess
import sys

import pytest

import bench
from workloads import make_workload_inputs, visible_pairs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    # The check runs before anything touches a GPU.
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flops_per_pair_add_up_to_the_step():
    # forward QK^T + PV (4d), dK/dV pass S, dP, dV, dK (8d), dQ pass dQ (2d): 14d per visible pair
    per_pair = bench.KERNEL_FLOPS_PER_PAIR_D
    assert per_pair["attn_sink_fwd_kernel"] + per_pair["attn_sink_bwd_dkdv_kernel"] + \
        per_pair["attn_sink_bwd_dq_kernel"] == 14


def test_source_digest_ignores_comments_but_not_code():
    code = 'int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */ const char* s = "a//b";\n'
    same = 'int f(int x) { return x + 1; }\nconst char* s = "a//b";  /* other */\n'
    other = 'int f(int x) { return x + 2; }\nconst char* s = "a//b";\n'
    assert bench._code_only(code) == bench._code_only(same)
    assert bench._code_only(code) != bench._code_only(other)
    assert '"a//b"' in bench._code_only(code)


@pytest.mark.gpu
def test_bench_line(monkeypatch, capsys):
    print("[gpu] bench.py --steps 10 --warmup 5 --settle-ms 100 --no-cpu-baseline --no-peaks (causal4k)", flush=True)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "10", "--warmup", "5", "--settle-ms", "100",
                                      "--no-cpu-baseline", "--no-peaks"])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    assert r["metric"] == bench.METRIC and r["unit"] == "TFLOP/s" and r["higher_is_better"] is True
    assert r["n_gpus"] == 1 and r["steps"] == 10 and r["warmup"] == 5
    assert r["dtype"] == "bf16" and r["data"] == "synthetic" and r["vs_baseline"] is None
    assert r["config"]["workload"] == "causal4k" and r["config"]["heads_q"] == 64 and r["config"]["heads_kv"] == 8
    assert r["settle"]["ms"] == 100.0 and r["settle"]["steps"] > 0
    inp = make_workload_inputs("causal4k", 0)
    flops = visible_pairs(inp.lengths, inp.causal, inp.window) * 64 * 14 * 64
    assert r["ms_per_step"] > 0
    assert r["value"] == pytest.approx(flops / (r["ms_per_step"] * 1e-3) / 1e12, rel=2e-3)
    rl = r["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == bench.MFMA_BF16_PEAK_TFLOPS
    assert rl["kernel"] in r["kernel_ms"]
    assert rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], abs=1e-4)
    assert 0 < rl["avg_launch_ms"] < r["ms_per_step"]
    assert rl["achieved"] == pytest.approx(rl["algorithmic_flops"] / (rl["avg_launch_ms"] * 1e-3) / 1e12, rel=2e-3)
    # every kernel of the step is in the breakdown, and together they fit in a step (events add a little)
    assert set(r["kernel_ms"]) == {"attn_sink_fwd_kernel", "attn_sink_bwd_dq_kernel", "attn_sink_bwd_dkdv_kernel",
                                   "attn_sink_bwd_finish_kernel"}
    assert sum(r["kernel_ms"].values()) < 1.2 * r["ms_per_step"]
