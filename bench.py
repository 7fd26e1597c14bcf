"""Benchmark: sink-attention forward + backward on one MI355X.

One step = attn_sink_fwd + attn_sink_bwd over one batch of synthetic GPT-OSS-shaped inputs that are
already resident in HBM. Default workload: 4096 tokens, 64 query heads sharing 8 KV heads,
head_dim 64, causal, bf16 inputs (the headline configuration).

    python bench.py [--gpus 1] [--steps 50] [--warmup 50] [--workload causal4k] [--no-cpu-baseline]

From idle, the first 20-40 steps of the 4k workload run up to 8% slower than the rest while the
GPU's clocks settle. So before the ``--warmup`` steps the script runs untimed steps for
``--settle-ms`` of wall time (300 by default; reported as ``settle`` in the output line); the timed
region is still exactly ``--steps`` steps.

``--workload decode32k`` (or decode32k_nq4, decode32k_window) times the inference-shaped decode
forward instead: a few new tokens per sequence against 16k-32k-token KV caches, reported as
algorithmic HBM GB/s (q, every cached K/V row a new token sees, out and LSE, each once).

Prints one JSON line. ``value`` is algorithmic TFLOP/s over the timed steps: 4*d FLOPs per visible
(query, key, head) in the forward (QK^T and PV) plus 10*d in the backward (S, dP, dV, dK, dQ);
recomputation and masked tile work are not counted. ``roofline`` describes the kernel with the
largest share of the step time (picked in a short pass between the warm-up and the timed steps,
each of its steps with events around one kernel only), timed with HIP events recorded around it,
on the stream the kernels run on, in every timed step; the per-kernel breakdown ``kernel_ms`` comes
from a pass of the same kind after the timed steps. The roofline is taken against the
bf16 MFMA peak for the causal workloads, and against HBM bandwidth (algorithmic bytes: each tensor
the kernel needs read or written once at its ABI dtype) for the banded window ones.
``measured_peaks`` gives a bf16 GEMM's and a device copy's rates on the same GPU, measured after the
timed steps, beside the spec peaks. ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample
of the same workload (with the host's CPU model and core count).

``--table`` times every training workload instead (forward and backward separately, median of
``--steps``) and prints one JSON line per workload with the max errors of that run against the
oracle and the oracle's time.

Each HIP event record costs about 3 us of GPU time on MI355X; events around every kernel of every
timed step added about 2.5% to a 4k step (and 10% to a decode call), so the timed steps carry only
the two events around the dominant kernel.

``--copy-probe-mib N`` also runs one device-to-device copy of N MiB before the timed steps, the
known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters of a ``rocprofv3 --pmc`` run.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import attention_learnable_sinks_attn_amd as asa  # noqa: E402
from workloads import (DECODE_WORKLOADS, WORKLOAD_NAMES, make_decode_workload_inputs, make_workload_inputs,  # noqa: E402
                       visible_pairs, workload)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
METRIC = "sink-attention fwd+bwd bf16 TFLOP/s + % MFMA peak (GQA 64/8, d=64, 4k causal)"

# Algorithmic FLOPs per visible (query, key, head) pair, per kernel, in units of head_dim:
# forward QK^T + PV; dK/dV pass S, dP, dV, dK; dQ pass dQ only (its S/dP recomputation is not counted).
KERNEL_FLOPS_PER_PAIR_D = {
    "attn_sink_fwd_kernel": 4,
    "attn_sink_bwd_dkdv_kernel": 8,
    "attn_sink_bwd_dq_kernel": 2,
    "attn_sink_bwd_finish_kernel": 0,
}


# HBM traffic of the dominant kernel, per launch, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) scaled by what the same counters read for the
# copy probe; valid only for kernel sources with the recorded digest.
TRAFFIC = {
    ("causal4k", "attn_sink_bwd_dkdv_kernel"): {"bytes": 146656344, "digest": "a3a1135a4abf74c7"},
    ("window4k", "attn_sink_bwd_dkdv_kernel"): {"bytes": 106700506, "digest": "a3a1135a4abf74c7"},
    ("window4k", "attn_sink_bwd_dq_kernel"): {"bytes": 213161614, "digest": "a3a1135a4abf74c7"},
    ("varlen_window", "attn_sink_bwd_dkdv_kernel"): {"bytes": 1708273888, "digest": "a3a1135a4abf74c7"},
    ("varlen_window", "attn_sink_bwd_dq_kernel"): {"bytes": 3648234371, "digest": "a3a1135a4abf74c7"},
    ("band4k", "attn_sink_bwd_dkdv_kernel"): {"bytes": 121165482, "digest": "a3a1135a4abf74c7"},
    ("band4k", "attn_sink_bwd_dq_kernel"): {"bytes": 213207535, "digest": "a3a1135a4abf74c7"},
    ("decode32k", "attn_sink_decode_partial_kernel"): {"bytes": 368469960, "digest": "a3a1135a4abf74c7"},
    ("causal4k", "attn_sink_fwd_kernel"): {"bytes": 114557098, "digest": "a3a1135a4abf74c7"},
    ("causal4k", "attn_sink_bwd_dq_kernel"): {"bytes": 221363909, "digest": "a3a1135a4abf74c7"},
    ("varlen_causal", "attn_sink_bwd_dkdv_kernel"): {"bytes": 8728681667, "digest": "a3a1135a4abf74c7"},
    ("long32k", "attn_sink_bwd_dkdv_kernel"): {"bytes": 35308073228, "digest": "a3a1135a4abf74c7"},
}


def _code_only(text: str) -> str:
    """C/C++ source without its comments and with whitespace runs collapsed (string literals kept)."""
    out = re.sub(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/',
                 lambda m: m.group(0) if m.group(0).startswith('"') else " ", text, flags=re.S)
    return " ".join(out.split())


def kernel_source_digest() -> str:
    """sha256 over the code (comments and layout ignored) of the HIP sources and headers the library
    is built from."""
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "attention_learnable_sinks_attn_amd", "csrc"), os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".h")):
                with open(os.path.join(d, name), encoding="utf-8") as f:
                    h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_bytes(name: str, T: int, hq: int, hkv: int, d: int) -> int:
    """Algorithmic HBM bytes of one launch: every tensor the kernel needs, read or written once."""
    q = T * hq * d * 2
    kv = 2 * T * hkv * d * 2
    rows = hq * T * 4  # one fp32 per (head, row): LSE, D
    o32 = T * hq * d * 4
    dkv32 = 2 * T * hkv * d * 4
    return {
        "attn_sink_fwd_kernel": q + kv + o32 + rows,
        "attn_sink_bwd_dkdv_kernel": 2 * q + kv + 2 * rows + dkv32,
        # q, dO, K, V and O in, LSE in, -LSE/scale and -D out, dQ out
        "attn_sink_bwd_dq_kernel": 2 * q + kv + 3 * rows + 2 * o32,
        "attn_sink_bwd_finish_kernel": dkv32,
    }[name]


class Hip:
    """The few HIP runtime calls needed for events on an arbitrary stream."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return e.value

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return out.value


def _oracle_threads() -> int:
    """Threads numpy's BLAS may use for the oracle's matrix products."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(inp, w, max_heads_kv: int):
    """Time the fp64 oracle (forward + backward) on the first `max_heads_kv` KV groups."""
    import numpy as np  # noqa: F401
    import oracle
    threads = _oracle_threads()
    G = w.hq // w.hkv
    hq_s = G * max_heads_kv
    q = inp.q[:, :hq_s]
    dout = inp.dout[:, :hq_s]
    k = inp.k[:, :max_heads_kv]
    v = inp.v[:, :max_heads_kv]
    sinks = inp.sinks[:hq_s]
    t0 = time.perf_counter()
    oracle.backward(q, k, v, sinks, dout, inp.cu_seqlens, inp.causal, inp.window, return_forward=True)
    dt = time.perf_counter() - t0
    flops = visible_pairs(inp.lengths, inp.causal, inp.window) * hq_s * 14 * w.d
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{w.name}: all {inp.total_tokens} rows of {max_heads_kv} KV group(s) ({hq_s} query heads), "
                     f"fwd+bwd in fp64 numpy, {dt:.2f} s"}
    res.update(cpu_info())
    return res


def decode_bytes(d, hq: int, hkv: int, out_bytes: int):
    """Algorithmic HBM bytes of one decode call: (q + every K/V row some new query sees) for the
    partial kernel, (out + lse) for the combine kernel."""
    cu_q, cu_k = d.cu_q.tolist(), d.cu_k.tolist()
    keys = 0
    for b in range(len(cu_q) - 1):
        nq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        if nq:
            keys += min(lk, d.window + nq - 1) if d.window > 0 else lk
    tq = cu_q[-1]
    dim = int(d.q.shape[2])
    return {"attn_sink_decode_partial_kernel": tq * hq * dim * 2 + 2 * keys * hkv * dim * 2,
            "attn_sink_decode_combine_kernel": tq * hq * dim * out_bytes + hq * tq * 4}


BREAKDOWN_STEPS = 5  # steps per kernel in the breakdown pass


def breakdown_source(n_kernels: int) -> str:
    return (f"a pass of {n_kernels} x {BREAKDOWN_STEPS} steps after the timed steps, step j with events "
            f"around kernel j % {n_kernels} only")


def settle(step, settle_ms: float) -> int:
    """Untimed steps for `settle_ms` of wall time (the host waits for the GPU every 8 steps, so it
    does not queue far ahead of it); returns how many ran."""
    n = 0
    t_end = time.perf_counter() + settle_ms / 1000.0
    while time.perf_counter() < t_end:
        step(None)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def run_timed(step, names, hip, warmup: int, steps: int):
    """`warmup` untimed steps; a short pass that picks the dominant kernel; exactly `steps` timed
    steps; then the breakdown pass.

    step(evs) runs one step; evs is None or a list of len(names) + 1 event handles (entries may be
    None), entry i recorded before kernel i and the last after the last kernel. Each event record
    costs about 3 us of GPU time, so no step carries more than two. The picking pass (2 steps per
    kernel) and the breakdown pass after the timed steps (BREAKDOWN_STEPS per kernel) time kernel
    j % n in their step j, with events around that kernel alone, so every kernel's samples spread
    over the whole pass. Each timed step carries the two events around the dominant kernel, whose
    average over the timed steps is its measured launch time. Returns (ms per step, wall seconds of
    the timed steps, per-kernel ms from the breakdown pass, dominant kernel, its ms over the timed
    steps)."""
    n = len(names)

    def evs_around(i, pair):
        e = [None] * (n + 1)
        e[i], e[i + 1] = pair
        return e

    def rotating_pass(per_kernel_steps):
        pairs = [(hip.event(), hip.event()) for _ in range(n * per_kernel_steps)]
        for j, pair in enumerate(pairs):
            step(evs_around(j % n, pair))
        torch.cuda.synchronize()
        return {nm: sum(hip.elapsed_ms(*pairs[j]) for j in range(i, len(pairs), n)) / per_kernel_steps
                for i, nm in enumerate(names)}

    for _ in range(warmup):
        step(None)
    pick = rotating_pass(2)
    dom = max(pick, key=pick.get)
    di = names.index(dom)
    timed = [(hip.event(), hip.event()) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for pair in timed:
        step(evs_around(di, pair))
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    dom_ms = sum(hip.elapsed_ms(a, b) for a, b in timed) / steps
    per_kernel = rotating_pass(BREAKDOWN_STEPS)
    return ms_step, wall, per_kernel, dom, dom_ms


def cpu_info() -> dict:
    """Host CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"cpu_model": model, "host_cores": len(os.sched_getaffinity(0))}


def measured_peaks(dev) -> dict:
    """Practical ceilings on this GPU, beside the spec peaks: a bf16 GEMM (torch.matmul, 8192^3,
    median of 10) and a device-to-device copy of 1 GiB (read + write bytes, median of 10)."""
    def median_ms(fn, reps=10):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    n = 8192
    x = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    y = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    z = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(x, y, out=z)
    gemm_ms = median_ms(lambda: torch.matmul(x, y, out=z))
    del x, y, z
    src = torch.empty((1 << 28,), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = median_ms(lambda: dst.copy_(src))
    nbytes = src.numel() * 4
    del src, dst
    torch.cuda.synchronize()
    res = {"bf16_gemm_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
           "copy_gbs": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1)}
    probe = os.path.join(ROOT, "attention_learnable_sinks_attn_amd", "libattn_sink_probe.so")
    how = "torch.matmul bf16 8192x8192x8192 and a 1 GiB device copy"
    if os.path.exists(probe):
        lib = ctypes.CDLL(probe)
        lib.attn_sink_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.attn_sink_probe_mfma.restype = ctypes.c_int
        blocks, iters = 2048, 4000
        buf = torch.empty((blocks * 256,), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream

        def run_probe():
            if lib.attn_sink_probe_mfma(buf.data_ptr(), blocks, iters, stream) != 0:
                raise RuntimeError("MFMA probe launch failed")

        run_probe()
        probe_ms = median_ms(run_probe)
        res["bf16_mfma_loop_tflops"] = round(blocks * 4 * iters * 8 * 32768 / (probe_ms * 1e-3) / 1e12, 1)
        how += ", and a register-only loop of 32x32x16 bf16 MFMAs on every SIMD (libattn_sink_probe.so)"
        del buf
    res["how"] = how + "; median of 10 each"
    return res


def bench_decode(args):
    """Decode forward (attn_sink_decode_fwd, bf16 output) over resident KV caches."""
    d = make_decode_workload_inputs(args.workload, args.seed)
    B = len(d.cu_k) - 1
    _, _, nq, hq, hkv, window = DECODE_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev).contiguous() for t in (d.q, d.k, d.v))
    sinks, cu_q, cu_k = d.sinks.to(dev), d.cu_q.to(dev), d.cu_k.to(dev)
    Tq = q.shape[0]
    out = torch.empty((Tq, hq, 64), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((hq, Tq), dtype=torch.float32, device=dev)
    ws = torch.empty((asa.decode_workspace_bytes(q, k, cu_q, d.max_q, d.max_k),), dtype=torch.uint8, device=dev)
    names = asa.decode_kernel_names()
    hip = Hip()

    def step(evs=None):
        asa.decode_fwd(q, k, v, sinks, cu_q, cu_k, d.max_q, d.max_k, window=window, out_dtype=torch.bfloat16,
                       out=out, lse=lse, workspace=ws, events=evs)

    n_settle = settle(step, args.settle_ms)
    ms_step, wall, per_kernel, dom, dom_ms = run_timed(step, names, hip, args.warmup, args.steps)
    kb = decode_bytes(d, hq, hkv, 2)
    total = sum(kb.values())
    gbs = total / (ms_step * 1e-3) / 1e9
    achieved = kb[dom] / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "avg_launch_ms": round(dom_ms, 4), "algorithmic_bytes": kb[dom]}
    rec = TRAFFIC.get((args.workload, dom))
    if rec is not None and rec["digest"] == kernel_source_digest():
        roofline["traffic"] = rec["bytes"]
        roofline["traffic_unit"] = "bytes per launch (HBM fetch + write)"
    res = {
        "metric": "sink-attention decode forward HBM GB/s (GQA 64/8, d=64, bf16 KV cache)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": n_settle}, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "seqs": B, "new_tokens": int(Tq), "cached_tokens": int(k.shape[0]),
                   "heads_q": hq, "heads_kv": hkv, "head_dim": 64, "window": window, "out_dtype": "bf16",
                   "seed": args.seed, "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(Tq / (ms_step * 1e-3), 1),
        "kernel_ms": {n: round(t, 4) for n, t in per_kernel.items()},
        "kernel_ms_from": breakdown_source(len(names)),
        "kernel_ms_sum": round(sum(per_kernel.values()), 4),
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        oracle.decode_forward(d.q, d.k, d.v, d.sinks, d.cu_q, d.cu_k, window)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": _oracle_threads(),
                               "kind": "oracle", "sample": f"{args.workload}: the whole batch ({B} sequences, "
                                                           f"{Tq} new tokens) in fp64 numpy, {dt:.2f} s"}
        res["cpu_baseline"].update(cpu_info())
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for this much wall time before the warm-up steps (clocks settle)")
    ap.add_argument("--workload", default="causal4k", choices=list(WORKLOAD_NAMES) + list(DECODE_WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-kv-groups", type=int, default=8)
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--no-peaks", action="store_true", help="skip the GEMM / copy ceiling measurements")
    ap.add_argument("--table", action="store_true",
                    help="results table: every training workload, t_fwd and t_bwd (median of --steps), max "
                         "errors and oracle time (one JSON line per workload)")
    ap.add_argument("--table-workloads", nargs="+", default=[w for w in WORKLOAD_NAMES])
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.table:
        bench_table(args)
        return
    if args.workload in DECODE_WORKLOADS:
        bench_decode(args)
        return
    w = workload(args.workload, args.seed)
    inp = make_workload_inputs(args.workload, args.seed)
    dev = torch.device("cuda:0")
    q, k, v, dout = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.dout))
    sinks = inp.sinks.to(dev)
    cu = inp.cu_seqlens.to(dev)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dq = torch.empty_like(out)
    dk = torch.empty((T, Hkv, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    dsinks = torch.empty((Hq,), dtype=torch.float32, device=dev)
    ws = torch.empty((asa.bwd_workspace_bytes(q, k, cu, inp.max_seqlen),), dtype=torch.uint8, device=dev)
    names = ["attn_sink_fwd_kernel"] + list(asa.bwd_kernel_names())

    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(evs=None):
        if evs is not None and evs[0] is not None:
            hip.record(evs[0], stream)
        bwd_ev = None if evs is None or all(e is None for e in evs[1:]) else evs[1:]
        asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, inp.causal, inp.window, out=out, lse=lse)
        asa.bwd(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, inp.causal, inp.window, dq=dq, dk=dk, dv=dv,
                dsinks=dsinks, workspace=ws, events=bwd_ev)

    n_settle = settle(step, args.settle_ms)
    ms_step, wall, per_kernel, dom, dom_ms = run_timed(step, names, hip, args.warmup, args.steps)

    pairs = visible_pairs(inp.lengths, inp.causal, inp.window) * Hq
    flops = pairs * 14 * d
    tflops = flops / (ms_step * 1e-3) / 1e12
    if inp.window > 0:  # banded: far less compute per byte than the ridge point
        dom_bytes = kernel_bytes(dom, T, Hq, Hkv, d)
        achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "avg_launch_ms": round(dom_ms, 4), "algorithmic_bytes": dom_bytes}
    else:
        dom_flops = pairs * KERNEL_FLOPS_PER_PAIR_D[dom] * d
        achieved = dom_flops / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "avg_launch_ms": round(dom_ms, 4), "algorithmic_flops": dom_flops}
    rec = TRAFFIC.get((w.name, dom))
    if rec is not None and rec["digest"] == kernel_source_digest():
        roofline["traffic"] = rec["bytes"]
        roofline["traffic_unit"] = "bytes per launch (HBM fetch + write)"
    # The headline metric names its own workload; any other workload is named in the metric too.
    metric = METRIC if w.name == "causal4k" else f"sink-attention fwd+bwd bf16 TFLOP/s ({w.name}: {w.description})"
    res = {
        "metric": metric, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": {"ms": args.settle_ms, "steps": n_settle}, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "tokens": int(T), "seqs": len(inp.lengths), "heads_q": int(Hq),
                   "heads_kv": int(Hkv), "head_dim": int(d), "causal": inp.causal, "window": inp.window,
                   "seed": args.seed, "parallelism": "none (1 GPU)"},
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "kernel_ms": {n: round(t, 4) for n, t in per_kernel.items()},
        "kernel_ms_from": breakdown_source(len(names)),
        "kernel_ms_sum": round(sum(per_kernel.values()), 4),
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
    }
    if not args.no_peaks:  # after the timed steps, so that they do not change the clocks those ran at
        peaks = measured_peaks(dev)
        res["measured_peaks"] = peaks
        if roofline["bound"] == "mfma":
            ceiling = peaks.get("bf16_mfma_loop_tflops", peaks["bf16_gemm_tflops"])
            roofline["frac_of_measured_peak"] = round(roofline["achieved"] / ceiling, 4)
        else:
            roofline["frac_of_measured_peak"] = round(roofline["achieved"] / peaks["copy_gbs"], 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_kv_groups)
    print(json.dumps(res), flush=True)


# ---- results table: every training workload, forward and backward timed separately ----------

def step_bytes(T: int, hq: int, hkv: int, d: int):
    """Algorithmic HBM bytes of a forward and of a backward: each tensor once at its ABI dtype
    (bf16 q, k, v, dO; fp32 O, LSE, dQ, dK, dV; the D workspace written and read once)."""
    q = T * hq * d * 2
    kv = 2 * T * hkv * d * 2
    rows = hq * T * 4
    o32 = T * hq * d * 4
    fwd = q + kv + o32 + rows
    bwd = 2 * q + kv + o32 + rows + o32 + 2 * T * hkv * d * 4 + 2 * rows
    return fwd, bwd


def oracle_leg(name, inp):
    """The cpu_baseline leg of the table: the fp64 oracle, timed, on the same inputs; its results
    also give the run's max errors. The whole oracle for the shorter workloads; one KV group (and
    dSink of every head from the stored oracle values in tests/golden) for varlen_causal and
    long32k, whose whole oracle takes minutes."""
    import numpy as np
    import oracle
    from workloads import input_digest
    Hq, Hkv = inp.q.shape[1], inp.k.shape[1]
    G = Hq // Hkv
    rb = 256 if inp.window > 0 else 1024
    if name in ("varlen_causal", "long32k"):
        grp = int(np.random.default_rng(11).integers(0, Hkv))
        heads = list(range(grp * G, (grp + 1) * G))
        t0 = time.perf_counter()
        r = oracle.backward(inp.q[:, heads], inp.k[:, grp:grp + 1], inp.v[:, grp:grp + 1], inp.sinks[heads],
                            inp.dout[:, heads], inp.cu_seqlens, inp.causal, inp.window, row_block=rb,
                            return_forward=True)
        dt = time.perf_counter() - t0
        with open(os.path.join(ROOT, "tests", "golden", f"dsink_{name}_seed0.json")) as f:
            gold = json.load(f)
        assert gold["input_digest"] == input_digest(inp)
        scope = f"KV group {grp} of {Hkv} (fwd+bwd); dSink of all heads from tests/golden"
        return r, dt, scope, heads, [grp], np.array(gold["dsink"])
    t0 = time.perf_counter()
    r = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, inp.causal, inp.window,
                        row_block=rb, return_forward=True)
    return r, time.perf_counter() - t0, "whole workload (fwd+bwd)", None, None, None


def bench_table(args):
    import numpy as np
    dev = torch.device("cuda:0")
    rows = []
    for name in args.table_workloads:
        inp = make_workload_inputs(name, args.seed)
        q, k, v, dout = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.dout))
        sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
        T, Hq, d = q.shape
        Hkv = k.shape[1]
        out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
        dq, dk = torch.empty_like(out), torch.empty((T, Hkv, d), dtype=torch.float32, device=dev)
        dv, ds = torch.empty_like(dk), torch.empty((Hq,), dtype=torch.float32, device=dev)
        ws = torch.empty((asa.bwd_workspace_bytes(q, k, cu, inp.max_seqlen),), dtype=torch.uint8, device=dev)

        def f():
            asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, inp.causal, inp.window, out=out, lse=lse)

        def b():
            asa.bwd(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, inp.causal, inp.window, dq=dq, dk=dk, dv=dv,
                    dsinks=ds, workspace=ws)

        settle(lambda _evs: (f(), b()), args.settle_ms)
        for _ in range(args.warmup):
            f()
            b()
        tf, tb = [], []
        for _ in range(args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            f()
            e[1].record()
            b()
            e[2].record()
            torch.cuda.synchronize()
            tf.append(e[0].elapsed_time(e[1]))
            tb.append(e[1].elapsed_time(e[2]))
        t_fwd, t_bwd = float(np.median(tf)), float(np.median(tb))
        pairs = visible_pairs(inp.lengths, inp.causal, inp.window) * Hq
        bf, bb = step_bytes(T, Hq, Hkv, d)
        total_ms = t_fwd + t_bwd
        row = {"workload": name, "tokens": int(T), "seqs": len(inp.lengths), "causal": inp.causal,
               "window": inp.window, "reps": args.steps, "t_fwd_ms": round(t_fwd, 4), "t_bwd_ms": round(t_bwd, 4),
               "tflops": round(pairs * 14 * d / (total_ms * 1e-3) / 1e12, 2),
               "pct_mfma_peak": round(100 * pairs * 14 * d / (total_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
               "gbs": round((bf + bb) / (total_ms * 1e-3) / 1e9, 1),
               "pct_hbm_peak": round(100 * (bf + bb) / (total_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        if not args.no_cpu_baseline:
            (rdq, rdk, rdv, rds, ro, rl), dt, scope, heads, kvh, gold_ds = oracle_leg(name, inp)
            hsel = slice(None) if heads is None else heads
            ksel = slice(None) if kvh is None else kvh
            errs = {}
            for nm, t, r in (("out", out[:, hsel], ro), ("dq", dq[:, hsel], rdq), ("dk", dk[:, ksel], rdk),
                             ("dv", dv[:, ksel], rdv), ("lse", lse[hsel], rl)):
                errs[nm] = float(np.max(np.abs(t.double().cpu().numpy() - r)))
            got_ds = ds.double().cpu().numpy()
            ref_ds = gold_ds if gold_ds is not None else rds
            errs["dsink_rel_max"] = float(np.max(np.abs(got_ds - ref_ds) / np.abs(ref_ds)))
            row["max_err"] = {n_: float(f"{e_:.3e}") for n_, e_ in errs.items()}
            row["oracle"] = {"seconds": round(dt, 2), "scope": scope, "threads": _oracle_threads(), **cpu_info()}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del q, k, v, dout, out, lse, dq, dk, dv, ds, ws
        torch.cuda.empty_cache()
    return rows


if __name__ == "__main__":
    main()
