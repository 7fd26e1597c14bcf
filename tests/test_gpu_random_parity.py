"""Seeded random sweep of the HIP path (through the C ABI) against the fp64 oracle.

Each case draws a packed batch with a mix of empty, single-token, ragged and multi-tile
sequences; a GQA ratio from 1 to 8; causal, causal-window, non-causal or band masks; an optional
softmax scale; and sinks that are ordinary, scaled x3, very large, or -inf on some heads. Every
element of O, LSE, dQ, dK, dV and dSink is compared, to the same tolerances as the fixed cases.
The draw depends only on the case index, so a failing case can be rerun by itself. The first 24
indices run at head_dim 64, twelve more at head_dim 128, and the draws of a wider sweep that once
failed are kept as regressions.
"""
import math

import numpy as np
import pytest

from test_gpu_parity import check_full, run_gpu, say
from workloads import make_inputs

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw_case(idx: int) -> dict:
    rng = np.random.default_rng(9000 + idx)
    B = int(rng.integers(1, 6))
    kinds = rng.choice(["empty", "one", "short", "tile", "long"], size=B, p=[0.1, 0.1, 0.3, 0.2, 0.3])
    lengths = []
    for k in kinds:
        if k == "empty":
            lengths.append(0)
        elif k == "one":
            lengths.append(1)
        elif k == "short":
            lengths.append(int(rng.integers(2, 64)))
        elif k == "tile":
            lengths.append(int(64 * rng.integers(1, 5)))
        else:
            lengths.append(int(rng.integers(65, 420)))
    if sum(lengths) == 0:
        lengths[0] = int(rng.integers(1, 200))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8]))
    causal = bool(rng.random() < 0.7)
    r = rng.random()
    if r < 0.4:
        window = 0
    elif r < 0.85:
        window = int(rng.integers(1, 300))
    else:
        window = int(max(lengths) + rng.integers(0, 50))  # at least the longest sequence
    scale = None if rng.random() < 0.6 else float(rng.uniform(0.04, 0.3))
    sinks = None
    sink_scale = 1.0
    r = rng.random()
    if r < 0.2:
        sink_scale = 3.0
    elif r < 0.4:  # some heads without a sink, some with a dominant one
        sinks = [float(x) for x in rng.normal(size=hkv * G)]
        for h in rng.choice(hkv * G, size=max(1, hkv * G // 3), replace=False):
            sinks[int(h)] = -math.inf if rng.random() < 0.5 else float(rng.uniform(8.0, 20.0))
    return dict(lengths=tuple(lengths), hq=hkv * G, hkv=hkv, causal=causal, window=window, scale=scale,
                sinks=sinks, sink_scale=sink_scale, seed=100 + idx)


def _run_case(idx, d):
    c = draw_case(idx)
    say(f"[gpu] random case {idx}: lengths={c['lengths']} hq={c['hq']} hkv={c['hkv']} causal={c['causal']} "
        f"window={c['window']} scale={c['scale']} sink_scale={c['sink_scale']} sinks={c['sinks']} d={d}")
    inp = make_inputs(c["lengths"], c["hq"], c["hkv"], d, causal=c["causal"], window=c["window"], seed=c["seed"],
                      sink_scale=c["sink_scale"], sinks_override=c["sinks"])
    check_full(inp, run_gpu(inp, c["scale"]), c["scale"])


@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_parity(idx):
    _run_case(idx, 64)


N_CASES_D128 = 12


@pytest.mark.parametrize("idx", range(1000, 1000 + N_CASES_D128))
def test_random_parity_d128(idx):
    _run_case(idx, 128)


# Draws from a wider sweep that once failed: 2092 (head_dim 128, softmax scale 0.262, three times
# the default, sinks x3) put dQ at 1.08e-2 while the forward's residual product started at a
# quarter of a row's probability mass; it starts at an eighth since.
@pytest.mark.parametrize("idx,d", [(2092, 128)])
def test_random_parity_regressions(idx, d):
    _run_case(idx, d)
