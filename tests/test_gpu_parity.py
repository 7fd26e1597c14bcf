"""Parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (GPU vs oracle): max-abs 1e-2 on O, dQ, dK, dV (fp32 outputs of bf16 ~N(0,1) inputs),
max-abs 1e-3 on the fp32 LSE, and 1e-2 relative error per head on dSink.

Small cases compare every element; they span several 64-row / 64-key tiles and end in ragged
tails. The full-size GPT-OSS-shaped workloads run in the same launch configuration the bench
times and are compared on sampled rows, keys and heads that the oracle evaluates one by one.
"""
import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import attention_learnable_sinks_attn_amd as asa
import oracle
from workloads import input_digest, make_inputs, make_workload_inputs

pytestmark = pytest.mark.gpu

TOL = {"out": 1e-2, "dq": 1e-2, "dk": 1e-2, "dv": 1e-2, "lse": 1e-3}
TOL_DSINK_REL = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(inp, scale=None, repeat_bwd=False):
    dev = torch.device("cuda:0")
    q, k, v, dout = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.dout))
    sinks = inp.sinks.to(dev)
    cu = inp.cu_seqlens.to(dev)
    out, lse = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, inp.causal, inp.window, scale)
    # The workspace starts as all-ones bytes (NaN as fp32): the backward must not read anything it
    # did not write in the same call.
    ws = torch.full((max(asa.bwd_workspace_bytes(q, k, cu, inp.max_seqlen), 1),), 255, dtype=torch.uint8, device=dev)
    dq, dk, dv, ds = asa.bwd(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, inp.causal, inp.window, scale,
                             workspace=ws)
    res = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dsinks": ds}
    if repeat_bwd:
        res2 = asa.bwd(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, inp.causal, inp.window, scale)
        res["again"] = res2
    torch.cuda.synchronize()
    return res


def maxabs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def check_dsink(got, ref, heads=None, label=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
    exact_zero = (ref == 0) & (got == 0)
    rel = np.where(exact_zero, 0.0, rel)
    worst = int(np.argmax(rel)) if rel.size else 0
    say(f"  dsinks{label}: max per-head rel err {rel.max() if rel.size else 0:.3e} (head {heads[worst] if heads else worst})")
    assert (rel <= TOL_DSINK_REL).all(), f"dSink rel err {rel.max():.3e} > {TOL_DSINK_REL}"


def check_full(inp, g, scale=None):
    out, lse = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, inp.causal, inp.window, scale)
    dq, dk, dv, ds = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, inp.causal,
                                     inp.window, scale)
    ref = {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    for name, r in ref.items():
        x = g[name].double().cpu().numpy()
        assert np.isfinite(x).all(), f"{name} has non-finite values"
        err = maxabs(x, r)
        say(f"  {name}: max-abs err {err:.3e} (max |ref| {np.abs(r).max() if r.size else 0:.3f})")
        assert err <= TOL[name], f"{name}: max-abs err {err:.3e} > {TOL[name]}"
    check_dsink(g["dsinks"].double().cpu().numpy(), ds)


SMALL_CASES = {
    # name: (lengths, hq, hkv, causal, window, extra)
    "mha_causal_ragged": ((300,), 2, 2, True, 0, {}),
    "gqa8_varlen_causal": ((130, 0, 1, 257, 64, 200), 16, 2, True, 0, {}),
    "varlen_empty_ends": ((0, 0, 70, 0, 33, 0), 4, 2, True, 0, {}),  # empty first, middle and last sequences
    "gqa2_window37": ((300, 77), 4, 2, True, 37, {}),
    "gqa8_window128": ((513, 129), 8, 1, True, 128, {}),
    "gqa4_noncausal": ((190, 65, 1), 8, 2, False, 0, {}),
    "mha_single_tokens": ((1, 1, 3, 1), 2, 2, True, 0, {}),
    "window_ge_len": ((150, 40), 4, 1, True, 1000, {}),
    "window_int_max": ((150, 40), 4, 1, True, 2**31 - 1, {}),  # no overflow in row + window
    "window1": ((97,), 2, 1, True, 1, {}),
    "sink_neg_inf_window": ((200, 63), 4, 2, True, 20, {"sinks": [-math.inf] * 4}),
    "sink_neg_inf_causal": ((130,), 2, 1, True, 0, {"sinks": [-math.inf, 0.5]}),
    "sink_plus20": ((160,), 2, 1, True, 0, {"sinks": [20.0, -3.0]}),
    "sinks_x3": ((300,), 4, 1, True, 0, {"sink_scale": 3.0}),
    "scale_0p07": ((140,), 2, 2, True, 0, {"scale": 0.07}),
    "exact_tiles": ((256, 128), 8, 8, True, 64, {}),
    "gqa3_causal": ((200, 70), 6, 2, True, 0, {}),
    "gqa6_window50": ((180,), 6, 1, True, 50, {}),
    # non-causal attention with a window: the symmetric band |i - j| < W
    "band_gqa4_w40": ((150, 70, 1), 8, 2, False, 40, {}),
    "band_gqa8_w128": ((513, 129), 8, 1, False, 128, {}),
    "band_w1": ((97, 33), 2, 1, False, 1, {}),
    "band_w_ge_len": ((150, 40), 4, 1, False, 1000, {}),
    "band_int_max": ((97, 33), 2, 1, False, 2**31 - 1, {}),
    "band_neg_inf_sinks": ((200, 63), 4, 2, False, 20, {"sinks": [-math.inf] * 4}),
    "band_exact_tiles": ((256, 128), 8, 8, False, 64, {}),
    # Enough (sequence, key block, KV head) triples that the dK/dV pass keeps each KV group's query
    # heads in one workgroup (two head streams, dK/dV written directly): 512 or more with a window,
    # 2048 or more without. Both reach that with 8 KV heads and 64 or 256 short sequences.
    "one_half_window": (tuple(int(x) for x in np.random.default_rng(3).integers(1, 130, 64)), 16, 8, True, 32, {}),
    "one_half_causal": (tuple(int(x) for x in np.random.default_rng(4).integers(1, 65, 256)), 16, 8, True, 0, {}),
    "one_half_band": (tuple(int(x) for x in np.random.default_rng(5).integers(1, 130, 64)), 16, 8, False, 20, {}),
}


def _small(name, d):
    lengths, hq, hkv, causal, window, extra = SMALL_CASES[name]
    inp = make_inputs(lengths, hq, hkv, d, causal=causal, window=window, seed=7,
                      sink_scale=extra.get("sink_scale", 1.0), sinks_override=extra.get("sinks"))
    scale = extra.get("scale")
    say(f"[gpu] small case {name}: lengths={lengths} hq={hq} hkv={hkv} causal={causal} window={window} d={d}")
    g = run_gpu(inp, scale)
    check_full(inp, g, scale)


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_small_parity(name):
    _small(name, 64)


# head_dim 128: rows of two 64-element panels, 32-key tiles, and the dK/dV pass at one wave per SIMD
D128_CASES = ["mha_causal_ragged", "gqa8_varlen_causal", "varlen_empty_ends", "gqa2_window37", "gqa8_window128",
              "gqa4_noncausal", "mha_single_tokens", "window_int_max", "sink_neg_inf_window", "sink_plus20",
              "sinks_x3", "scale_0p07", "gqa3_causal", "gqa6_window50", "band_gqa4_w40", "band_exact_tiles",
              "exact_tiles", "one_half_window", "one_half_causal", "one_half_band"]


@pytest.mark.parametrize("name", D128_CASES)
def test_small_parity_d128(name):
    _small(name, 128)


def test_tiny_workload_full_parity():
    inp = make_workload_inputs("tiny")
    say("[gpu] workload tiny (1 head, 128 tokens, causal)")
    check_full(inp, run_gpu(inp))


@pytest.mark.parametrize("hq,hkv,window", [(4, 2, 0), (3, 1, 0), (3, 1, 16)])
def test_empty_input(hq, hkv, window):
    # Even GQA ratios split the dK/dV pass's heads into halves and reduce dSink in the finish
    # kernel; odd ones reduce it at the end of the dK/dV launch. Either way every head's dSink is
    # written (zero) although no row exists: the buffer starts as NaN.
    say(f"[gpu] empty input (T = 0), heads {hq}/{hkv}, window {window}")
    inp = make_inputs((0,), hq, hkv, 64, window=window, seed=1)
    g = run_gpu(inp)
    assert g["out"].numel() == 0
    assert torch.all(g["dsinks"] == 0)
    dev = torch.device("cuda:0")
    q, k, v, dout = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.dout))
    ds = torch.full((hq,), float("nan"), device=dev)
    asa.bwd(q, k, v, inp.sinks.to(dev), g["out"], g["lse"], dout, inp.cu_seqlens.to(dev), inp.max_seqlen,
            inp.causal, inp.window, dsinks=ds)
    torch.cuda.synchronize()
    assert torch.all(ds == 0)


@pytest.mark.parametrize("nseq", [256, 257])
def test_dsink_reduction_either_side_of_the_fold_limit(nseq):
    # 8 KV heads x nseq sequences of at most 64 tokens (one key block each), window 32, so no head
    # halves: 2048 key-block workgroups reduce dSink at the end of the dK/dV launch, 2056 leave it
    # to the finish kernel. Every element against the oracle.
    rng = np.random.default_rng(nseq)
    lengths = tuple(int(x) for x in rng.integers(1, 65, nseq - 1)) + (64,)
    say(f"[gpu] dSink reduction at the fold limit: {nseq} sequences x 8 KV heads, {sum(lengths)} tokens")
    inp = make_inputs(lengths, 16, 8, 64, causal=True, window=32, seed=nseq)
    check_full(inp, run_gpu(inp))


@pytest.mark.parametrize("d,hq,hkv", [(64, 16, 2), (128, 16, 2), (64, 3, 1)])
def test_backward_is_deterministic(d, hq, hkv):
    # GQA 8 splits the dK/dV pass's heads into halves (finish kernel); GQA 3 does not, and its
    # small launch also reduces dSink itself.
    inp = make_inputs((700, 333), hq, hkv, d, causal=True, window=0, seed=2)
    say(f"[gpu] determinism: two backward calls on the same inputs, d={d}, heads {hq}/{hkv}")
    g = run_gpu(inp, repeat_bwd=True)
    for a, b in zip((g["dq"], g["dk"], g["dv"], g["dsinks"]), g["again"]):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the bench times.
#  * causal4k, window4k, band4k, varlen_window: every element of every output against the whole
#    oracle (seconds of fp64 CPU work);
#  * varlen_causal, long32k: every element of one whole KV group (its 8 query heads' O, LSE, dQ and
#    dSink, every key of its dK and dV, key block 0 included, whose sums run over every row of the
#    sequence), and dSink of all 64 heads against stored oracle values (tests/golden,
#    make_dsink_golden.py), since a head's dSink needs that head's softmax over every row.
# ---------------------------------------------------------------------------------------------

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _oracle_row_block(inp):
    # With a window, row blocks of 256 keep the oracle's key range per block near the window; the
    # arithmetic of each row is the same for any blocking.
    return 256 if inp.window > 0 else 1024


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["causal4k", "window4k", "band4k", "varlen_window", "causal4k_d128",
                                  "causal4k_sharp"])
def test_full_size_every_element(name):
    inp = make_workload_inputs(name)
    say(f"[gpu] full-size workload {name}, every element: T={inp.total_tokens} B={len(inp.lengths)} "
        f"window={inp.window}")
    g = run_gpu(inp)
    rb = _oracle_row_block(inp)
    dq, dk, dv, ds, out, lse = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens,
                                               inp.causal, inp.window, row_block=rb, return_forward=True)
    compare_all(g, {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, ds)


def compare_all(g, ref, ds_ref, heads=None, kv_heads=None):
    """Every element of the GPU outputs (restricted to `heads` / `kv_heads` when given) against the
    oracle's."""
    sel = {"out": heads, "dq": heads, "lse": heads, "dk": kv_heads, "dv": kv_heads}
    for name, r in ref.items():
        t = g[name]
        idx = sel[name]
        if idx is not None:
            ix = torch.tensor(idx, device=t.device)
            t = t.index_select(0 if name == "lse" else 1, ix)
        x = t.double().cpu().numpy()
        assert np.isfinite(x).all(), f"{name} has non-finite values"
        err = maxabs(x, r)
        say(f"  {name} {tuple(x.shape)}: max-abs err {err:.3e} (max |ref| {np.abs(r).max() if r.size else 0:.3f})")
        assert err <= TOL[name], f"{name}: max-abs err {err:.3e} > {TOL[name]}"
    got = g["dsinks"].double().cpu().numpy()
    check_dsink(got if heads is None else got[heads], ds_ref, heads, label="" if heads is None else f" {heads}")


def load_golden_dsink(name, inp):
    path = os.path.join(GOLDEN, f"dsink_{name}_seed0.json")
    with open(path) as f:
        rec = json.load(f)
    assert rec["input_digest"] == input_digest(inp), f"{path} was computed from other inputs"
    return np.array(rec["dsink"], dtype=np.float64), np.array(rec["abs_terms"], dtype=np.float64)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["varlen_causal", "long32k"])
def test_full_size_one_kv_group(name):
    inp = make_workload_inputs(name)
    Hq, Hkv = inp.q.shape[1], inp.k.shape[1]
    G = Hq // Hkv
    grp = int(np.random.default_rng(11).integers(0, Hkv))
    heads = list(range(grp * G, (grp + 1) * G))
    say(f"[gpu] full-size workload {name}: T={inp.total_tokens} B={len(inp.lengths)}; every element of KV group "
        f"{grp} (query heads {heads[0]}..{heads[-1]}), dSink of all {Hq} heads")
    g = run_gpu(inp)
    dq, dk, dv, ds, out, lse = oracle.backward(inp.q[:, heads], inp.k[:, grp:grp + 1], inp.v[:, grp:grp + 1],
                                               inp.sinks[heads], inp.dout[:, heads], inp.cu_seqlens, inp.causal,
                                               inp.window, return_forward=True)
    compare_all(g, {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, ds, heads=heads, kv_heads=[grp])
    ref, terms = load_golden_dsink(name, inp)
    check_dsink(g["dsinks"].double().cpu().numpy(), ref, list(range(Hq)), label=" (all heads, stored oracle values)")
    say(f"  dsinks: condition number sum|terms|/|sum| up to {np.max(terms / np.abs(ref)):.1f}")


def _sample_rows(cu, rng, n):
    T = int(cu[-1])
    rows = set(rng.integers(0, T, size=n).tolist())
    for b in range(len(cu) - 1):          # sequence boundaries and tails
        a, e = int(cu[b]), int(cu[b + 1])
        if e > a:
            rows.update({a, e - 1})
    return sorted(rows)[: n + 2 * (len(cu) - 1)]


def _sample_keys(cu, causal, window, rng, n):
    keys = set()
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        L = e - a
        if L == 0:
            continue
        if window > 0 or L <= 4096:
            keys.update({a, e - 1, a + int(rng.integers(0, L))})
        else:                                   # causal long sequence: keys near the end are cheap
            keys.update({e - 1, e - 1 - int(rng.integers(0, 64))})
    keys = sorted(keys)
    if len(keys) > n:
        keys = sorted(rng.choice(keys, size=n, replace=False).tolist())
    return keys


def test_longest_sequence_131072_sampled():
    """One 128k-token sequence of one GQA group (8 query heads, 1 KV head; one rank's share under
    8-way head parallelism): 4096 query blocks per head and 2048 key blocks, the longest rows the
    tests run. dSink is left to the 32k case (its oracle needs every row of the head)."""
    inp = make_inputs((131072,), 8, 1, 64, causal=True, window=0, seed=8)
    say(f"[gpu] longest sequence: T={inp.total_tokens}")
    check_sampled(inp, run_gpu(inp), dsink=False, n_rows=8, n_heads=3)


def check_sampled(inp, g, dsink=True, n_rows=24, n_heads=6):
    cu = inp.cu_seqlens.numpy()
    rng = np.random.default_rng(123)
    Hq, Hkv = inp.q.shape[1], inp.k.shape[1]
    for name_t in ("out", "lse", "dq", "dk", "dv", "dsinks"):
        assert torch.isfinite(g[name_t]).all(), f"{name_t} has non-finite values"
    rows = _sample_rows(cu, rng, n_rows)
    heads = sorted(rng.choice(Hq, size=n_heads, replace=False).tolist())
    o_ref, l_ref = oracle.forward_rows(inp.q, inp.k, inp.v, inp.sinks, cu, rows, heads, inp.causal, inp.window)
    dq_ref = oracle.dq_rows(inp.q, inp.k, inp.v, inp.sinks, inp.dout, cu, rows, heads, inp.causal, inp.window)
    idx_r = torch.tensor(rows)
    idx_h = torch.tensor(heads)
    o_gpu = g["out"].cpu()[idx_r][:, idx_h].double().numpy()
    l_gpu = g["lse"].cpu()[idx_h][:, idx_r].double().numpy()
    dq_gpu = g["dq"].cpu()[idx_r][:, idx_h].double().numpy()
    for label, x, r, tol in (("out", o_gpu, o_ref, TOL["out"]), ("lse", l_gpu, l_ref, TOL["lse"]),
                             ("dq", dq_gpu, dq_ref, TOL["dq"])):
        err = maxabs(x, r)
        say(f"  {label} ({len(rows)} rows x {len(heads)} heads): max-abs err {err:.3e}")
        assert err <= tol
    keys = _sample_keys(cu, inp.causal, inp.window, rng, 12)
    kvh = sorted(rng.choice(Hkv, size=min(2, Hkv), replace=False).tolist())
    dk_ref, dv_ref = oracle.dkdv_keys(inp.q, inp.k, inp.v, inp.sinks, inp.dout, cu, keys, kvh, inp.causal,
                                      inp.window)
    idx_k = torch.tensor(keys)
    idx_g = torch.tensor(kvh)
    for label, t, r in (("dk", g["dk"], dk_ref), ("dv", g["dv"], dv_ref)):
        x = t.cpu()[idx_k][:, idx_g].double().numpy()
        err = maxabs(x, r)
        say(f"  {label} ({len(keys)} keys x {len(kvh)} kv heads): max-abs err {err:.3e}")
        assert err <= TOL[label]
    if not dsink:
        return
    ds_heads = heads[:2]
    ds_ref = oracle.dsink_heads(inp.q, inp.k, inp.v, inp.sinks, inp.dout, cu, ds_heads, inp.causal, inp.window)
    check_dsink(g["dsinks"].cpu().double().numpy()[ds_heads], ds_ref, ds_heads, label=f" (heads {ds_heads})")


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 77), (False, 0), (False, 40)])
def test_forward_bf16_output_is_rounded_fp32_output(causal, window):
    """out_dtype bf16: the same fp32 result rounded to nearest even; LSE unchanged."""
    inp = make_inputs((300, 1, 129), 8, 2, 64, causal=causal, window=window, seed=4)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
    say(f"[gpu] bf16 forward output: causal={causal} window={window}")
    o32, l32 = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, causal, window)
    o16, l16 = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, causal, window, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32)


@pytest.mark.parametrize("hq,hkv,kernel", [(16, 2, "attn_sink_bwd_dkdv_kernel"), (3, 1, "attn_sink_bwd_dkdv_kernel"),
                                            (3, 1, "attn_sink_bwd_finish_kernel")])
def test_timed_backward_records_only_the_given_events(hq, hkv, kernel):
    """attn_sink_bwd_timed with NULL entries: results unchanged, the given events bracket a kernel.
    With an odd GQA ratio (no head halves, a small launch) the dK/dV launch reduces dSink and the
    finish kernel is not launched: its events are recorded back to back."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(2):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    inp = make_inputs((300, 77), hq, hkv, 64, causal=True, window=0, seed=5)
    dev = torch.device("cuda:0")
    q, k, v, dout = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.dout))
    sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
    say(f"[gpu] timed backward, heads {hq}/{hkv}, events around {kernel} only")
    out, lse = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, True, 0)
    ref = asa.bwd(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, True, 0)
    names = list(asa.bwd_kernel_names())
    i = names.index(kernel)
    events = [None] * (len(names) + 1)
    events[i], events[i + 1] = evs
    got = asa.bwd(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, True, 0, events=events)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) == 0
    if kernel == "attn_sink_bwd_dkdv_kernel":
        assert ms.value > 0.0
    else:
        assert ms.value >= 0.0
    for e in evs:
        hip.hipEventDestroy(e)
