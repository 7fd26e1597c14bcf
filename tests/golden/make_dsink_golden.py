"""Writes the stored dL/dS_h references of the long full-size workloads (every query head).

dL/dS_h = -sum_i P_{i,h} D_i sums over every row of every packed sequence (nmedialink.com
"惊爆！GPT-OSS-20B强化学习，训练速度狂飙、超稳定！", section "反向传播的实现", simplified
equation), so one head's value needs that head's full softmax over the whole workload. For the
32768-token and the packed 16-sequence workloads that is minutes of fp64 CPU work per run, too
slow to repeat inside a GPU test; this script computes it once with ``oracle.dsink_heads`` alone
(inputs from ``workloads``) and stores, per head, the value and sum_i |P_{i,h} D_i| (the
conditioning of the sum). Each file also records a digest of the input tensors, which the tests
check before comparing, so that a stored value is only ever used for the inputs it was computed
from.

    python tests/golden/make_dsink_golden.py [--workloads long32k varlen_causal] [--jobs 8]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def golden_path(name: str, seed: int) -> str:
    return os.path.join(HERE, f"dsink_{name}_seed{seed}.json")


def _heads_job(args):
    name, seed, heads, threads = args
    os.environ["OMP_NUM_THREADS"] = str(threads)
    os.environ["OPENBLAS_NUM_THREADS"] = str(threads)
    import oracle
    from workloads import make_workload_inputs
    inp = make_workload_inputs(name, seed)
    vals, terms = oracle.dsink_heads(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, list(heads),
                                     inp.causal, inp.window, return_terms=True)
    return list(heads), [float(x) for x in vals], [float(x) for x in terms]


def make(name: str, seed: int, jobs: int) -> dict:
    from workloads import input_digest, make_workload_inputs, workload
    w = workload(name, seed)
    inp = make_workload_inputs(name, seed)
    digest = input_digest(inp)
    del inp
    chunks = [list(range(h, w.hq, jobs)) for h in range(jobs)]
    chunks = [c for c in chunks if c]
    vals = [0.0] * w.hq
    terms = [0.0] * w.hq
    t0 = time.perf_counter()
    ctx = __import__("multiprocessing").get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=len(chunks), mp_context=ctx) as ex:
        for heads, v, t in ex.map(_heads_job, [(name, seed, c, 1) for c in chunks]):
            for h, a, b in zip(heads, v, t):
                vals[h], terms[h] = a, b
            print(f"  {name}: heads {heads} done ({time.perf_counter() - t0:.0f} s)", flush=True)
    return {
        "about": ("dL/dS_h of every query head, from oracle.dsink_heads (fp64 NumPy) on the seeded workload "
                  "inputs; written by tests/golden/make_dsink_golden.py"),
        "workload": name, "seed": seed, "input_digest": digest,
        "dsink": vals, "abs_terms": terms, "oracle_seconds": round(time.perf_counter() - t0, 1),
        "oracle_processes": len(chunks),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", nargs="+", default=["long32k", "varlen_causal"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--jobs", type=int, default=8)
    args = ap.parse_args()
    for name in args.workloads:
        rec = make(name, args.seed, args.jobs)
        with open(golden_path(name, args.seed), "w") as f:
            json.dump(rec, f, indent=1)
        print(f"wrote {golden_path(name, args.seed)} ({rec['oracle_seconds']} s)", flush=True)


if __name__ == "__main__":
    main()
