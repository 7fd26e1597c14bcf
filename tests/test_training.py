"""Training integration: position ids -> cu_seqlens (CPU) and autograd through the HIP kernels (GPU).

The GPU test compares the gradients that ``loss.backward()`` leaves on q, k, v and the sink
parameter with the fp64 oracle's backward of the same inputs and upstream gradient.
"""
import pytest
import torch

from attention_learnable_sinks_attn_amd.training import cu_seqlens_from_position_ids


def test_cu_seqlens_from_position_ids():
    pos = torch.tensor([0, 1, 2, 0, 0, 1, 2, 3, 0, 1])
    cu, maxlen = cu_seqlens_from_position_ids(pos)
    assert cu.tolist() == [0, 3, 4, 8, 10] and cu.dtype == torch.int32
    assert maxlen == 4
    cu, maxlen = cu_seqlens_from_position_ids(torch.zeros(0, dtype=torch.int64))
    assert cu.tolist() == [0] and maxlen == 0


@pytest.mark.parametrize("bad", [[1, 2, 3], [0, 1, 3], [0, 2], [0, 1, 1]])
def test_cu_seqlens_from_position_ids_rejects(bad):
    with pytest.raises(ValueError):
        cu_seqlens_from_position_ids(torch.tensor(bad))


@pytest.mark.gpu
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 40), (False, 0), (False, 40)])
def test_autograd_matches_oracle(causal, window):
    import oracle
    from attention_learnable_sinks_attn_amd.training import SinkAttention
    from workloads import make_inputs

    inp = make_inputs((150, 0, 70), 8, 2, 64, causal=causal, window=window, seed=11)
    dev = torch.device("cuda:0")
    pos = torch.cat([torch.arange(n) for n in inp.lengths if n > 0])
    cu, maxlen = cu_seqlens_from_position_ids(pos)
    # zero-length sequences leave no position ids; the packed rows are the same
    q = inp.q.to(dev).requires_grad_(True)
    k = inp.k.to(dev).requires_grad_(True)
    v = inp.v.to(dev).requires_grad_(True)
    layer = SinkAttention(8, 2, causal=causal, window=window).to(dev)
    with torch.no_grad():
        layer.sinks.copy_(inp.sinks.to(dev))
    out = layer(q, k, v, cu.to(dev), maxlen)
    dout = inp.dout.to(dev).float()
    (out * dout).sum().backward()

    rdq, rdk, rdv, rds, rout, _ = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens,
                                                  causal, window, return_forward=True)
    assert abs(out.detach().cpu().double().numpy() - rout).max() <= 1e-2
    # gradients come back in the inputs' dtype (bf16): allow its storage rounding on top of 1e-2
    for name, g, r in (("dq", q.grad, rdq), ("dk", k.grad, rdk), ("dv", v.grad, rdv)):
        assert g.dtype == torch.bfloat16
        err = abs(g.detach().cpu().double().numpy() - r).max()
        assert err <= 1e-2 + abs(r).max() * 2 ** -8, (name, err)
    ds = layer.sinks.grad.detach().cpu().double().numpy()
    rel = (abs(ds - rds) / abs(rds).clip(1e-12)).max()
    assert rel <= 1e-2, rel
