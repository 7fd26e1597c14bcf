"""Seeded random sweep of both decode forwards (through the C ABI).

Each draw packs a few sequences with a mix of empty, one-token, short and longer caches, takes up
to a few dozen of each sequence's last tokens as the new queries (within the ABI's limit on
(new token, query head) pairs per KV head), and varies the GQA ratio, the window, the softmax
scale, the sinks (ordinary, x3, -inf or dominant on some heads) and the output dtype. For every
draw the split-KV decode is compared with the fp64 oracle to the training tolerances, and the
order-preserving decode must equal the training forward's rows bit for bit (and pass the same
oracle check). The draw depends only on its index, so a failing one can be rerun by itself.
"""
import math

import numpy as np
import pytest
import torch

import attention_learnable_sinks_attn_amd as asa
from test_gpu_decode import check_against_oracle, say
from workloads import last_rows, make_decode_inputs, make_inputs

pytestmark = pytest.mark.gpu

N_DRAWS = 16
N_DRAWS_D128 = 8


def draw_decode_case(idx: int) -> dict:
    rng = np.random.default_rng(7000 + idx)
    B = int(rng.integers(1, 7))
    kinds = rng.choice(["empty", "one", "short", "mid", "long"], size=B, p=[0.1, 0.1, 0.25, 0.35, 0.2])
    lengths = []
    for k in kinds:
        lengths.append({"empty": 0, "one": 1}.get(k) if k in ("empty", "one") else
                       int(rng.integers(2, 65) if k == "short" else rng.integers(65, 700) if k == "mid"
                           else rng.integers(700, 3000)))
    if sum(lengths) == 0:
        lengths[0] = int(rng.integers(1, 300))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    max_new = max(1, min(32, 1024 // G))
    nq = [int(min(L, rng.integers(0, max_new + 1) if rng.random() < 0.3 else rng.integers(0, 5))) for L in lengths]
    if sum(nq) == 0:
        nq[int(np.argmax(lengths))] = 1
    r = rng.random()
    window = 0 if r < 0.5 else (int(rng.integers(1, 400)) if r < 0.9 else int(max(lengths) + rng.integers(0, 50)))
    scale = None if rng.random() < 0.6 else float(rng.uniform(0.04, 0.3))
    sinks, sink_scale = None, 1.0
    r = rng.random()
    if r < 0.2:
        sink_scale = 3.0
    elif r < 0.4:
        sinks = [float(x) for x in rng.normal(size=hkv * G)]
        for h in rng.choice(hkv * G, size=max(1, hkv * G // 3), replace=False):
            sinks[int(h)] = -math.inf if rng.random() < 0.5 else float(rng.uniform(8.0, 20.0))
    out_dtype = torch.bfloat16 if rng.random() < 0.4 else torch.float32
    return dict(lengths=tuple(lengths), nq=tuple(nq), hq=hkv * G, hkv=hkv, window=window, scale=scale,
                sinks=sinks, sink_scale=sink_scale, out_dtype=out_dtype, seed=300 + idx)


def run_decode_case(idx: int, d: int):
    c = draw_decode_case(idx)
    say(f"[gpu] random decode {idx}: lengths={c['lengths']} nq={c['nq']} hq={c['hq']} hkv={c['hkv']} "
        f"window={c['window']} scale={c['scale']} sink_scale={c['sink_scale']} sinks={c['sinks']} "
        f"out={c['out_dtype']} d={d}")
    inp = make_inputs(c["lengths"], c["hq"], c["hkv"], d, causal=True, window=c["window"], seed=c["seed"],
                      sink_scale=c["sink_scale"], sinks_override=c["sinks"])
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v))
    sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
    rows, cu_q = last_rows(inp.cu_seqlens, c["nq"])
    rows_t = torch.tensor(rows, dtype=torch.long)
    qd = q[rows_t.to(dev)].contiguous()
    max_q = max(c["nq"])
    out_s, lse_s = asa.decode_fwd(qd, k, v, sinks, cu_q.to(dev), cu, max_q, inp.max_seqlen, window=c["window"],
                                  softmax_scale=c["scale"], out_dtype=c["out_dtype"])
    out_o, lse_o = asa.decode_fwd_ordered(qd, k, v, sinks, cu_q.to(dev), cu, max_q, inp.max_seqlen,
                                          window=c["window"], softmax_scale=c["scale"], out_dtype=c["out_dtype"])
    out_t, lse_t = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, True, c["window"], softmax_scale=c["scale"],
                           out_dtype=c["out_dtype"])
    torch.cuda.synchronize()
    dd = make_decode_inputs(c["lengths"], c["nq"], c["hq"], c["hkv"], d, window=c["window"], seed=0)
    dd.q, dd.k, dd.v, dd.sinks = inp.q[rows_t], inp.k, inp.v, inp.sinks
    dd.cu_q, dd.cu_k = cu_q, inp.cu_seqlens
    say("  split-KV decode:")
    check_against_oracle(dd, out_s, lse_s, c["scale"])
    say("  order-preserving decode:")
    check_against_oracle(dd, out_o, lse_o, c["scale"])
    assert torch.equal(out_o, out_t[rows_t.to(dev)]), "ordered decode out differs from the training forward's rows"
    assert torch.equal(lse_o, lse_t[:, rows_t.to(dev)]), "ordered decode lse differs from the training forward's rows"


@pytest.mark.parametrize("idx", range(N_DRAWS))
def test_random_decode(idx):
    run_decode_case(idx, 64)


@pytest.mark.parametrize("idx", range(1000, 1000 + N_DRAWS_D128))
def test_random_decode_d128(idx):
    run_decode_case(idx, 128)
