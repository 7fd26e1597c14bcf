"""Parity of the HIP decode (inference-shaped) forward, through the C ABI, against the fp64 oracle,
and its consistency with the training forward.

Tolerances against the oracle are those of the training forward: max-abs 1e-2 on O and 1e-3 on the
fp32 LSE; a bf16 O may differ by half a bf16 ulp more (its own rounding, which alone exceeds 1e-2
where |O| >= 4). Small cases compare every element and cover several key chunks
with ragged tails, GQA groups of 1 to 8, per-sequence numbers of new tokens (0 included), a
sliding window, sinks at -inf, sequences made only of new tokens and an empty batch. The
full-size cases run the 8-sequence, 16k-32k-key GPT-OSS-shaped caches in the launch
configuration the bench times and compare every output.

Train/inference consistency: the decode forward and the training forward compute the same rows
with the same bf16 rounding of P but sum the keys in another order and against another running
maximum, so they agree to rounding, not bitwise; the test bounds the difference well inside the
parity tolerance (CONSIST_TOL).
"""
import sys

import numpy as np
import pytest
import torch

import attention_learnable_sinks_attn_amd as asa
import oracle
from workloads import last_rows, make_decode_inputs, make_decode_workload_inputs, make_inputs

pytestmark = pytest.mark.gpu

TOL_OUT, TOL_LSE = 1e-2, 1e-3
CONSIST_TOL = {"out": 4e-3, "lse": 1e-4}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_decode(d, out_dtype=torch.float32, scale=None):
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev).contiguous() for t in (d.q, d.k, d.v))
    out, lse = asa.decode_fwd(q, k, v, d.sinks.to(dev), d.cu_q.to(dev), d.cu_k.to(dev), d.max_q, d.max_k,
                              window=d.window, softmax_scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


def bf16_half_ulp(x):
    """Half the bf16 spacing at |x| (8 significant bits): what storing x in bf16 may cost."""
    e = np.floor(np.log2(np.maximum(np.abs(x), np.finfo(np.float32).tiny)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_against_oracle(d, out, lse, scale=None, ref=None):
    """O and LSE of a decode call against the oracle (``ref``: its (out, lse), if already computed)."""
    ro, rl = ref if ref is not None else oracle.decode_forward(d.q, d.k, d.v, d.sinks, d.cu_q, d.cu_k, d.window,
                                                               scale)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert np.isfinite(o).all(), "out has non-finite values"
    eo = float(np.max(np.abs(o - ro))) if o.size else 0.0
    # A bf16 output also carries its own rounding of the fp32 value y it was made from, at most half
    # a bf16 ulp of y, which is at most half an ulp of the stored output (7.8e-3 for |O| in [2, 4),
    # more above): the tolerance bounds the error beyond it.
    slack = bf16_half_ulp(o) if out.dtype == torch.bfloat16 else np.zeros_like(ro)
    eo_beyond = float(np.max(np.abs(o - ro) - slack)) if o.size else 0.0
    fin = np.isfinite(rl)
    assert (np.isfinite(l) == fin).all(), "LSE -inf pattern differs"
    el = float(np.max(np.abs(l[fin] - rl[fin]))) if fin.any() else 0.0
    say(f"  out: max-abs err {eo:.3e} ({eo_beyond:.3e} beyond the output's own rounding)   lse: max-abs err {el:.3e}")
    assert eo_beyond <= TOL_OUT, f"out: max-abs err {eo_beyond:.3e} beyond the output rounding > {TOL_OUT}"
    assert el <= TOL_LSE, f"lse: max-abs err {el:.3e} > {TOL_LSE}"


# name: (cache lengths, new tokens per sequence, Hq, Hkv, window, kwargs)
SMALL = {
    "g8_nq1": ((100, 37, 260, 1), 1, 8, 1, 0, {}),
    "g8_nq4_bf16": ((300, 64, 129), 4, 16, 2, 0, {"out_dtype": torch.bfloat16}),
    "g4_mixed_nq": ((200, 70, 5, 333), (2, 0, 5, 8), 8, 2, 0, {}),
    "g2_window50": ((400, 90, 33), 3, 4, 2, 50, {}),
    "g1_nq32": ((300, 40), (32, 17), 2, 2, 0, {}),
    "g8_window1": ((129, 64), 2, 8, 1, 1, {"out_dtype": torch.bfloat16}),
    "all_new_tokens": ((5, 8, 3), (5, 8, 3), 8, 2, 0, {}),
    "neg_inf_sinks": ((150, 77), 2, 8, 1, 0, {"sinks": float("-inf")}),
    "big_sinks": ((257, 31), 1, 16, 2, 0, {"sink_scale": 3.0}),
    "scale_0p3": ((190,), 4, 8, 1, 0, {"scale": 0.3}),
    "window_ge_len": ((70, 20), 3, 8, 2, 500, {}),
    "window_int_max": ((70, 20), 3, 8, 2, 2**31 - 1, {}),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_small(name):
    lengths, nq, hq, hkv, window, kw = SMALL[name]
    kw = dict(kw)
    out_dtype = kw.pop("out_dtype", torch.float32)
    scale = kw.pop("scale", None)
    sink_value = kw.pop("sinks", None)
    d = make_decode_inputs(lengths, nq, hq, hkv, window=window, seed=11, **kw)
    if sink_value is not None:
        d.sinks.fill_(sink_value)
    say(f"decode {name}: Lk={lengths} nq={nq} heads {hq}/{hkv} window={window} out={out_dtype}")
    out, lse = run_decode(d, out_dtype, scale)
    assert out.dtype == out_dtype
    check_against_oracle(d, out, lse, scale)


D128_SMALL = ["g8_nq1", "g4_mixed_nq", "g2_window50", "neg_inf_sinks", "g8_nq4_bf16", "g1_nq32", "all_new_tokens"]


@pytest.mark.parametrize("name", D128_SMALL)
def test_decode_small_d128(name):
    lengths, nq, hq, hkv, window, kw = SMALL[name]
    kw = dict(kw)
    out_dtype = kw.pop("out_dtype", torch.float32)
    sink_value = kw.pop("sinks", None)
    d = make_decode_inputs(lengths, nq, hq, hkv, 128, window=window, seed=12, **kw)
    if sink_value is not None:
        d.sinks.fill_(sink_value)
    say(f"decode {name} d=128: Lk={lengths} nq={nq} heads {hq}/{hkv} window={window} out={out_dtype}")
    out, lse = run_decode(d, out_dtype)
    assert out.shape[2] == 128
    check_against_oracle(d, out, lse)


def test_decode_full_size_d128():
    lengths = np.random.default_rng(0).integers(16384, 32768, 8, endpoint=True)
    d = make_decode_inputs(lengths, 1, 64, 8, 128, seed=0)
    say(f"decode 8 x 16k-32k cached tokens, d=128: Lk={[int(x) for x in lengths]}")
    out, lse = run_decode(d, torch.bfloat16)
    check_against_oracle(d, out, lse)


def test_decode_empty_batch():
    d = make_decode_inputs((10, 20), 0, 8, 1, seed=1)
    say("decode: no new tokens")
    out, lse = run_decode(d)
    assert out.shape == (0, 8, 64) and lse.shape == (8, 0)


@pytest.mark.parametrize("nq,hq,hkv,window", [(5, 8, 1, 0), (16, 64, 8, 0), (9, 16, 2, 40), (31, 32, 1, 0)])
def test_decode_several_column_groups(nq, hq, hkv, window):
    # more (new token, query head) pairs per KV head than one 32-column MFMA block holds
    d = make_decode_inputs((300, 70, 1029), nq, hq, hkv, window=window, seed=2)
    say(f"decode: {nq} new tokens x {hq // hkv} heads per KV head, window {window}")
    out, lse = run_decode(d)
    check_against_oracle(d, out, lse)


def test_decode_rejects_too_many_columns():
    d = make_decode_inputs((200, 250), 129, 8, 1, seed=1)  # 129 new tokens x 8 heads > 1024 columns
    say("decode: unsupported max_q * group")
    with pytest.raises(asa.AttnSinkError) as e:
        run_decode(d)
    assert e.value.code == -3


@pytest.mark.parametrize("name", ["decode32k", "decode32k_nq4", "decode32k_window"])
def test_decode_full_size(name):
    """Both decode forwards on caches of 16k-32k tokens per sequence, every element against the oracle."""
    d = make_decode_workload_inputs(name, seed=0)
    say(f"decode {name}: Lk={[int(x) for x in (d.cu_k[1:] - d.cu_k[:-1])]} max_q={d.max_q}")
    ref = oracle.decode_forward(d.q, d.k, d.v, d.sinks, d.cu_q, d.cu_k, d.window, None)
    out, lse = run_decode(d, torch.bfloat16)
    say("  split-KV decode:")
    check_against_oracle(d, out, lse, ref=ref)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev).contiguous() for t in (d.q, d.k, d.v))
    out_o, lse_o = asa.decode_fwd_ordered(q, k, v, d.sinks.to(dev), d.cu_q.to(dev), d.cu_k.to(dev), d.max_q, d.max_k,
                                          window=d.window, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    say("  order-preserving decode:")
    check_against_oracle(d, out_o, lse_o, ref=ref)


@pytest.mark.parametrize("window,d", [(0, 64), (128, 64), (0, 128)])
def test_train_inference_consistency(window, d):
    """Training forward over whole packed sequences vs the decode forward over their last tokens."""
    lengths = (1000, 3000, 517, 64, 2049)
    nq = (1, 4, 3, 2, 4)
    inp = make_inputs(lengths, 64, 8, d, causal=True, window=window, seed=5)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v))
    sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
    say(f"consistency: lengths {lengths} new tokens {nq} window {window} d={d}")
    out_t, lse_t = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, True, window)
    rows, cu_q = last_rows(inp.cu_seqlens, nq)
    rows_t = torch.tensor(rows, device=dev)
    out_d, lse_d = asa.decode_fwd(q[rows_t].contiguous(), k, v, sinks, cu_q.to(dev), cu, max(nq), inp.max_seqlen,
                                  window=window)
    torch.cuda.synchronize()
    do = (out_d - out_t[rows_t]).abs().max().item()
    dl = (lse_d - lse_t[:, rows_t]).abs().max().item()
    say(f"  training vs decode: out max-abs diff {do:.3e}, lse max-abs diff {dl:.3e}")
    assert do <= CONSIST_TOL["out"] and dl <= CONSIST_TOL["lse"]


ORDERED_CASES = {
    # name: (lengths, new tokens per sequence, Hq, Hkv, d, window, sinks kwargs, out dtype)
    "g8_causal": ((1000, 3000, 517, 64, 2049), (1, 4, 3, 2, 4), 64, 8, 64, 0, {}, torch.float32),
    "g8_window128": ((1000, 3000, 517, 64, 2049), (1, 4, 3, 2, 4), 64, 8, 64, 128, {}, torch.float32),
    "g8_sinks_x3_bf16": ((700, 33, 1500), (2, 1, 5), 16, 2, 64, 0, {"sink_scale": 3.0}, torch.bfloat16),
    "g4_window7_neg_inf": ((300, 129, 64), (3, 2, 1), 8, 2, 64, 7, {"sinks_override": [float("-inf")] * 8},
                           torch.float32),
    "g1_many_tokens": ((200, 90), (40, 17), 2, 2, 64, 0, {}, torch.float32),
    "d128_causal": ((1000, 3000, 517, 64, 2049), (1, 4, 3, 2, 4), 64, 8, 128, 0, {}, torch.float32),
    "d128_window50": ((900, 77), (3, 2), 16, 2, 128, 50, {}, torch.float32),
}


@pytest.mark.parametrize("name", sorted(ORDERED_CASES))
def test_ordered_decode_equals_training_forward_bitwise(name):
    """attn_sink_decode_fwd_ordered reproduces the training forward's rows bit for bit (the opt-in
    answer to the train/inference mismatch); the default split-KV decode agrees to rounding."""
    lengths, nq, hq, hkv, d, window, kw, out_dtype = ORDERED_CASES[name]
    inp = make_inputs(lengths, hq, hkv, d, causal=True, window=window, seed=6, **kw)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v))
    sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
    say(f"ordered decode {name}: lengths {lengths} new tokens {nq} heads {hq}/{hkv} d={d} window {window}")
    out_t, lse_t = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, True, window, out_dtype=out_dtype)
    rows, cu_q = last_rows(inp.cu_seqlens, nq)
    rows_t = torch.tensor(rows, device=dev)
    out_d, lse_d = asa.decode_fwd_ordered(q[rows_t].contiguous(), k, v, sinks, cu_q.to(dev), cu, max(nq),
                                          inp.max_seqlen, window=window, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref_o, ref_l = out_t[rows_t], lse_t[:, rows_t]
    diff = (out_d.float() - ref_o.float()).abs().max().item()
    say(f"  ordered decode vs training forward: out max-abs diff {diff:.3e}, "
        f"equal: out {torch.equal(out_d, ref_o)}, lse {torch.equal(lse_d, ref_l)}")
    assert torch.equal(out_d, ref_o)
    assert torch.equal(lse_d, ref_l)
    # and against the oracle, like the split-KV decode
    dd = make_decode_inputs(tuple(lengths), nq, hq, hkv, d, window=window, seed=0)
    dd.q, dd.k, dd.v, dd.sinks = inp.q[torch.tensor(rows)], inp.k, inp.v, inp.sinks
    dd.cu_q, dd.cu_k = cu_q, inp.cu_seqlens
    check_against_oracle(dd, out_d, lse_d)


def test_ordered_decode_handles_empty_sequences():
    inp = make_inputs((0, 300, 1, 0, 70), 8, 2, 64, causal=True, seed=9)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v))
    sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
    say("ordered decode with empty sequences and sequences without new tokens")
    out_t, lse_t = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, True, 0)
    nq = (0, 3, 1, 0, 0)
    rows, cu_q = last_rows(inp.cu_seqlens, nq)
    rows_t = torch.tensor(rows, device=dev)
    out_d, lse_d = asa.decode_fwd_ordered(q[rows_t].contiguous(), k, v, sinks, cu_q.to(dev), cu, max(nq),
                                          inp.max_seqlen)
    torch.cuda.synchronize()
    assert torch.equal(out_d, out_t[rows_t]) and torch.equal(lse_d, lse_t[:, rows_t])


def test_decode_timed_records_only_the_given_events():
    """attn_sink_decode_fwd_timed with a NULL entry: results unchanged, the given events bracket the
    partial kernel."""
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
    d = make_decode_inputs((700, 1500, 90), 2, 8, 2, seed=3)
    dev = torch.device("cuda:0")
    args = ((d.q.to(dev), d.k.to(dev), d.v.to(dev), d.sinks.to(dev), d.cu_q.to(dev), d.cu_k.to(dev), d.max_q,
             d.max_k))
    say("[gpu] timed decode with events around the partial kernel only")
    ref = asa.decode_fwd(*args)
    got = asa.decode_fwd(*args, events=[evs[0], evs[1], None])
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) == 0
    assert ms.value > 0.0
    for e in evs:
        hip.hipEventDestroy(e)
