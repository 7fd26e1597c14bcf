"""Training integration: sink attention as a differentiable PyTorch op with learnable sinks.

``sink_attention`` wraps the library's forward and backward in a ``torch.autograd.Function``
(argument marshalling only; both passes run in the HIP kernels), so that q, k, v and the
per-head sink logits receive gradients through ordinary ``loss.backward()``. ``SinkAttention``
holds the sinks as an ``nn.Parameter``, one logit per query head, as in the attention-sink
layer of nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section "GPT-OSS中的带注意力槽的注意力机制".

Packed batches are described by ``cu_seqlens``; ``cu_seqlens_from_position_ids`` derives them
from per-token position ids that restart at 0 for every packed sequence (the padding-free packing
of the same page, section "结合Flash Attention V3的序列并行技术").

Dtypes: q, k, v are bf16; the output is fp32. The upstream gradient is rounded to bf16 before the
backward (the kernels take dO in bf16); dQ, dK, dV are computed in fp32 and returned in the
inputs' dtype, dSink in fp32.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import bwd, fwd

__all__ = ["sink_attention", "SinkAttention", "cu_seqlens_from_position_ids"]


class _SinkAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, sinks, cu_seqlens, max_seqlen, causal, window, softmax_scale):
        out, lse = fwd(q, k, v, sinks, cu_seqlens, max_seqlen, causal=causal, window=window,
                       softmax_scale=softmax_scale)
        ctx.save_for_backward(q, k, v, sinks, out, lse, cu_seqlens)
        ctx.cfg = (max_seqlen, causal, window, softmax_scale)
        ctx.mark_non_differentiable(lse)  # an output for inspection; no gradient flows through it
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, sinks, out, lse, cu_seqlens = ctx.saved_tensors
        max_seqlen, causal, window, softmax_scale = ctx.cfg
        dq, dk, dv, dsinks = bwd(q, k, v, sinks, out, lse, dout.to(torch.bfloat16).contiguous(), cu_seqlens,
                                 max_seqlen, causal=causal, window=window, softmax_scale=softmax_scale)
        return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dsinks.to(sinks.dtype),
                None, None, None, None, None)


def sink_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: torch.Tensor,
                   cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = True, window: int = 0,
                   softmax_scale: Optional[float] = None, return_lse: bool = False):
    """Differentiable sink attention over a packed batch.

    q [T, Hq, D], k / v [T, Hkv, D] bf16 (CUDA; D = 64 or 128); sinks [Hq] fp32; cu_seqlens [B+1] int32 on the
    same device. Returns out [T, Hq, D] fp32 (and lse [Hq, T] fp32 if ``return_lse``).
    """
    out, lse = _SinkAttentionFn.apply(q.contiguous(), k.contiguous(), v.contiguous(), sinks.contiguous(),
                                      cu_seqlens, int(max_seqlen), bool(causal), int(window), softmax_scale)
    return (out, lse) if return_lse else out


class SinkAttention(torch.nn.Module):
    """Attention core with one learnable sink logit per query head (initialised to ``init``)."""

    def __init__(self, num_heads_q: int, num_heads_kv: int, causal: bool = True, window: int = 0,
                 softmax_scale: Optional[float] = None, init: float = 0.0):
        super().__init__()
        if num_heads_q % num_heads_kv:
            raise ValueError("num_heads_q must be a multiple of num_heads_kv")
        self.num_heads_q, self.num_heads_kv = num_heads_q, num_heads_kv
        self.causal, self.window, self.softmax_scale = causal, window, softmax_scale
        self.sinks = torch.nn.Parameter(torch.full((num_heads_q,), float(init), dtype=torch.float32))

    def forward(self, q, k, v, cu_seqlens, max_seqlen):
        return sink_attention(q, k, v, self.sinks, cu_seqlens, max_seqlen, causal=self.causal, window=self.window,
                              softmax_scale=self.softmax_scale)


def cu_seqlens_from_position_ids(position_ids: torch.Tensor):
    """(cu_seqlens int32 [B+1], max_seqlen) from 1-D position ids of a packed batch.

    Every packed sequence's positions run 0, 1, 2, ...; a new sequence starts wherever the
    position is 0. Raises if the ids do not have that form.
    """
    pos = position_ids.reshape(-1).to(torch.int64)
    T = pos.numel()
    if T == 0:
        return torch.zeros(1, dtype=torch.int32, device=position_ids.device), 0
    starts = torch.nonzero(pos == 0).reshape(-1)
    if starts.numel() == 0 or int(starts[0]) != 0:
        raise ValueError("position ids must start a sequence (position 0) at token 0")
    cu = torch.cat([starts, torch.tensor([T], device=pos.device)])
    lengths = cu[1:] - cu[:-1]
    expected = torch.arange(T, device=pos.device) - torch.repeat_interleave(cu[:-1], lengths)
    if not torch.equal(pos, expected):
        raise ValueError("position ids must count 0, 1, 2, ... within every packed sequence")
    return cu.to(torch.int32), int(lengths.max())
