"""attn_sink_bwd_noalloc (the backward whose workspace is a static per-GPU scratch array) against
attn_sink_bwd with a caller workspace, through the C ABI: two calls in a row, the second on a
smaller input, each compared with the allocating entry point (bitwise: both run the same kernels
with the same launch configuration) and with the fp64 oracle to the parity tolerances. Also the
host-side rejection of shapes whose workspace exceeds the scratch array."""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import attention_learnable_sinks_attn_amd as asa
import oracle
from workloads import make_inputs

TOL = {"dq": 1e-2, "dk": 1e-2, "dv": 1e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """Host-only: the workspace size check runs before any HIP call."""
    lib = asa.load_library()
    P = 0x10000
    s = asa.Shape(262144, 1, 262144, 64, 8, 64, 0.0, 0)
    assert lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s)) > asa.NOALLOC_SCRATCH_BYTES
    rc = lib.attn_sink_bwd_noalloc(P, P, P, P, P, P, P, 1, 0, P, ctypes.byref(s), P, P, P, P, None)
    assert rc == -9
    assert b"scratch" in lib.attn_sink_strerror(-9)
    s = asa.Shape(4096, 1, 4096, 64, 8, 64, 0.0, 0)
    assert lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s)) <= asa.NOALLOC_SCRATCH_BYTES
    assert lib.attn_sink_bwd_noalloc(P, P, P, P, P, P, P, 1, 0, P, ctypes.byref(s), None, P, P, P, None) == -1


def _one_call(inp, label):
    dev = torch.device("cuda:0")
    q, k, v, dout = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.dout))
    sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
    say(f"[gpu] no-alloc backward, {label}: lengths={inp.lengths} hq={q.shape[1]} hkv={k.shape[1]} "
        f"causal={inp.causal} window={inp.window}")
    out, lse = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, inp.causal, inp.window)
    ref = asa.bwd(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, inp.causal, inp.window)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    # outputs start as NaN: every element must be written by the call
    got = [torch.full((T, Hq, d), float("nan"), device=dev), torch.full((T, Hkv, d), float("nan"), device=dev),
           torch.full((T, Hkv, d), float("nan"), device=dev), torch.full((Hq,), float("nan"), device=dev)]
    asa.bwd_noalloc(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, inp.causal, inp.window,
                    dq=got[0], dk=got[1], dv=got[2], dsinks=got[3])
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dsinks"), ref, got):
        assert torch.equal(a, b), f"{name}: no-alloc result differs from attn_sink_bwd"
    rdq, rdk, rdv, rds = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, inp.causal,
                                         inp.window)
    for name, x, r in (("dq", got[0], rdq), ("dk", got[1], rdk), ("dv", got[2], rdv)):
        err = float(np.max(np.abs(x.double().cpu().numpy() - r)))
        say(f"  {name}: max-abs err vs oracle {err:.3e}")
        assert err <= TOL[name]
    rel = np.abs(got[3].double().cpu().numpy() - rds) / np.abs(rds)
    say(f"  dsinks: max per-head rel err {rel.max():.3e}")
    assert (rel <= 1e-2).all()


@pytest.mark.gpu
def test_noalloc_matches_allocating_backward_twice():
    # first a larger problem (two head halves and their partial sums in the scratch), then a smaller
    # one with a window (one head half): the second must not see anything the first left behind
    _one_call(make_inputs((700, 333, 1), 16, 2, 64, causal=True, window=0, seed=21), "call 1")
    _one_call(make_inputs((150, 40), 8, 2, 64, causal=True, window=37, seed=22), "call 2 (smaller)")
