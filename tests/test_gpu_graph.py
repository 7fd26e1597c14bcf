"""The forward, backward and decode calls can be captured into a HIP graph (through torch's CUDA
graph API) and replayed: every replay matches the eager results bit for bit (the kernels are
deterministic, enqueue no memset, and allocate nothing)."""
import sys

import pytest
import torch

import attention_learnable_sinks_attn_amd as asa
from workloads import make_decode_inputs, make_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("hq,hkv", [(16, 2), (3, 1)])
def test_training_step_graph_replays_match_eager(hq, hkv):
    # GQA 8: the backward's three kernels (head halves, finish); GQA 3: two (the dK/dV launch
    # reduces dSink).
    inp = make_inputs((700, 1, 333), hq, hkv, causal=True, window=0, seed=21)
    dev = torch.device("cuda:0")
    q, k, v, dout = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.dout))
    sinks, cu = inp.sinks.to(dev), inp.cu_seqlens.to(dev)
    T, Hq, d = q.shape
    ws = torch.empty((asa.bwd_workspace_bytes(q, k, cu, inp.max_seqlen),), dtype=torch.uint8, device=dev)
    say("[gpu] graph capture: eager reference")
    ref_out, ref_lse = asa.fwd(q, k, v, sinks, cu, inp.max_seqlen)
    ref = asa.bwd(q, k, v, sinks, ref_out, ref_lse, dout, cu, inp.max_seqlen, workspace=ws)
    torch.cuda.synchronize()

    out = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dq = torch.empty_like(out)
    dk = torch.empty((T, k.shape[1], d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ds = torch.empty((Hq,), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    graph = torch.cuda.CUDAGraph()
    say("[gpu] graph capture: capturing fwd + bwd")
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            asa.fwd(q, k, v, sinks, cu, inp.max_seqlen, out=out, lse=lse)
            asa.bwd(q, k, v, sinks, out, lse, dout, cu, inp.max_seqlen, dq=dq, dk=dk, dv=dv, dsinks=ds, workspace=ws)
    torch.cuda.current_stream(dev).wait_stream(side)
    for rep in range(3):
        for t in (out, lse, dq, dk, dv, ds):
            t.fill_(float("nan"))
        # eager work of the program between replays
        scratch = (q.float() * 2.0).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}: comparing with eager")
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        for name, x, r in zip(("dq", "dk", "dv", "dsinks"), (dq, dk, dv, ds), ref):
            assert torch.equal(x, r), name
        del scratch


def test_decode_graph_replays_match_eager():
    dd = make_decode_inputs((3000, 517, 64), 4, 16, 2, window=0, seed=3)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev).contiguous() for t in (dd.q, dd.k, dd.v))
    sinks, cu_q, cu_k = dd.sinks.to(dev), dd.cu_q.to(dev), dd.cu_k.to(dev)
    ws = torch.empty((asa.decode_workspace_bytes(q, k, cu_q, dd.max_q, dd.max_k),), dtype=torch.uint8, device=dev)
    say("[gpu] decode graph capture: eager reference")
    ref_out, ref_lse = asa.decode_fwd(q, k, v, sinks, cu_q, cu_k, dd.max_q, dd.max_k, out_dtype=torch.bfloat16,
                                      workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            asa.decode_fwd(q, k, v, sinks, cu_q, cu_k, dd.max_q, dd.max_k, out_dtype=torch.bfloat16, out=out, lse=lse,
                           workspace=ws)
    torch.cuda.current_stream(dev).wait_stream(side)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  decode replay {rep}: comparing with eager")
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
