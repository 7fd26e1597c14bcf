"""Seeded synthetic inputs for sink attention (shared by the HIP path's tests/bench and the oracle).

This module only draws and rounds random numbers and packs sequence offsets. It holds none of
the method's arithmetic, so both the oracle and the HIP path may use it without sharing code.

Recipe (every config, one seed per run):
  * sequence lengths first (varlen configs only): numpy ``default_rng(seed).integers(512, 8192,
    size=16, endpoint=True)``; fixed-shape configs are a single sequence;
  * then a ``torch.Generator().manual_seed(seed)`` draws float32 N(0, 1) in the order
    q [T, Hq, d], k [T, Hkv, d], v [T, Hkv, d], dout [T, Hq, d], sinks [Hq];
  * q, k, v, dout are rounded to bfloat16 (round-to-nearest-even); sinks stay float32 and are
    multiplied by ``sink_scale`` (3 for the 32k long-context workload); ``q_scale`` (4 for the
    sharp-attention variant of the 4k workload) multiplies q before its rounding.

The pages' own workloads are GPT-OSS-20B RL runs (GSM8K, ReTool, VerifyIf) on packed
rollouts; no dataset or weight is used here. These GPT-OSS-shaped N(0, 1) tensors stand in
for them: 64 query heads sharing 8 KV heads, head_dim 64, 1/sqrt(64) softmax scale, and
(for varlen) 16 packed sequences of uniform length in [512, 8192].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple
    hq: int
    hkv: int
    d: int = 64
    causal: bool = True
    window: int = 0
    sink_scale: float = 1.0
    q_scale: float = 1.0
    description: str = ""

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.lengths)) if self.lengths else 0


def _varlen_lengths(seed: int) -> tuple:
    return tuple(int(x) for x in np.random.default_rng(seed).integers(512, 8192, size=16, endpoint=True))


def workload(name: str, seed: int = 0) -> Workload:
    """The five GPT-OSS-shaped workloads (six runs: the varlen batch runs causal and windowed)."""
    if name == "tiny":
        return Workload(name, (128,), 1, 1, description="1 head, 128 tokens, causal")
    if name == "causal4k":
        return Workload(name, (4096,), 64, 8, description="4096 tokens, GQA 64/8, d=64, causal")
    if name == "window4k":
        return Workload(name, (4096,), 64, 8, window=128,
                        description="4096 tokens, GQA 64/8, d=64, causal sliding window 128")
    if name == "varlen_causal":
        return Workload(name, _varlen_lengths(seed), 64, 8,
                        description="16 packed sequences, lengths U[512,8192], GQA 64/8, causal")
    if name == "varlen_window":
        return Workload(name, _varlen_lengths(seed), 64, 8, window=128,
                        description="16 packed sequences, lengths U[512,8192], GQA 64/8, window 128")
    if name == "band4k":
        return Workload(name, (4096,), 64, 8, causal=False, window=128,
                        description="4096 tokens, GQA 64/8, d=64, non-causal band |i - j| < 128")
    if name == "long32k":
        return Workload(name, (32768,), 64, 8, sink_scale=3.0,
                        description="32768 tokens, GQA 64/8, causal, sinks x3")
    if name == "causal4k_sharp":
        return Workload(name, (4096,), 64, 8, q_scale=4.0,
                        description="causal4k with q x4 (score std 4: peaked rows, like a trained layer's)")
    if name == "causal4k_d128":
        return Workload(name, (4096,), 64, 8, d=128,
                        description="4096 tokens, GQA 64/8, head_dim 128, causal (beyond the pages' d = 64)")
    raise KeyError(name)


WORKLOAD_NAMES = ("tiny", "causal4k", "window4k", "varlen_causal", "varlen_window", "long32k", "band4k",
                  "causal4k_d128", "causal4k_sharp")


@dataclass
class Inputs:
    q: torch.Tensor        # [T, Hq, d] bf16 (CPU)
    k: torch.Tensor        # [T, Hkv, d] bf16
    v: torch.Tensor        # [T, Hkv, d] bf16
    dout: torch.Tensor     # [T, Hq, d] bf16
    sinks: torch.Tensor    # [Hq] fp32
    cu_seqlens: torch.Tensor  # [B+1] int32
    lengths: tuple
    causal: bool
    window: int
    max_seqlen: int
    meta: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return torch.from_numpy(cu.astype(np.int32))


def make_inputs(lengths, hq: int, hkv: int, d: int = 64, *, causal: bool = True, window: int = 0,
                seed: int = 0, sink_scale: float = 1.0, sinks_override: Optional[List[float]] = None,
                zero_q: bool = False, q_scale: float = 1.0) -> Inputs:
    """Draw one batch following the recipe above. ``zero_q`` / ``sinks_override`` build the
    special inputs some pins need (uniform scores, S_h = -inf); they only replace drawn values.
    ``q_scale`` multiplies q before its bf16 rounding (sharper softmax rows)."""
    lengths = tuple(int(x) for x in lengths)
    T = int(sum(lengths))
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((T, hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((T, hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((T, hkv, d), generator=g, dtype=torch.float32)
    dout = torch.randn((T, hq, d), generator=g, dtype=torch.float32)
    sinks = torch.randn((hq,), generator=g, dtype=torch.float32) * float(sink_scale)
    if q_scale != 1.0:
        q = q * float(q_scale)
    if sinks_override is not None:
        sinks = torch.tensor(list(sinks_override), dtype=torch.float32)
        assert sinks.shape == (hq,)
    if zero_q:
        q = torch.zeros_like(q)
    return Inputs(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=v.to(torch.bfloat16),
                  dout=dout.to(torch.bfloat16), sinks=sinks.contiguous(), cu_seqlens=cu_from_lengths(lengths),
                  lengths=lengths, causal=bool(causal), window=int(window),
                  max_seqlen=max(lengths) if lengths else 0,
                  meta=dict(hq=hq, hkv=hkv, d=d, seed=seed, sink_scale=sink_scale, q_scale=q_scale))


def make_workload_inputs(name: str, seed: int = 0) -> Inputs:
    w = workload(name, seed)
    inp = make_inputs(w.lengths, w.hq, w.hkv, w.d, causal=w.causal, window=w.window, seed=seed,
                      sink_scale=w.sink_scale, q_scale=w.q_scale)
    inp.meta["workload"] = name
    return inp


def input_digest(inp: Inputs) -> str:
    """sha256 (first 32 hex digits) over the exact bytes of q, k, v, dout, sinks and cu_seqlens, so
    that a stored reference is only used for the inputs it was computed from."""
    import hashlib
    h = hashlib.sha256()
    for t in (inp.q, inp.k, inp.v, inp.dout, inp.sinks, inp.cu_seqlens):
        t = t.detach().contiguous().cpu()
        h.update(str(t.dtype).encode() + str(tuple(t.shape)).encode())
        h.update(t.view(torch.uint8).numpy().tobytes())
    return h.hexdigest()[:32]


def visible_pairs(lengths, causal: bool, window: int) -> int:
    """Number of (query, key) pairs a query may attend to, summed over sequences (one head)."""
    total = 0
    for L in lengths:
        L = int(L)
        if not causal:
            if window and window > 0:  # band i - W < j < i + W inside [0, L)
                i = np.arange(L, dtype=np.int64)
                total += int((np.minimum(i + int(window), L) - np.maximum(i - int(window) + 1, 0)).sum())
            else:
                total += L * L
        elif window and window > 0:
            W = int(window)
            m = min(L, W)
            # rows 0..m-1 see i+1 keys; rows m..L-1 see W keys
            total += m * (m + 1) // 2 + (L - m) * W
        else:
            total += L * (L + 1) // 2
    return total


# ---- inference-shaped (decode) inputs ----------------------------------------------------------
# Recipe: cache lengths Lk_b drawn first with numpy.default_rng(seed).integers(lo, hi, B,
# endpoint=True); then a torch.Generator(seed) draws fp32 N(0,1) in the order k, v (all Tk cached
# tokens), q (the Nq new tokens of every sequence, which are its last Nq tokens), sinks; q, k, v
# are rounded to bf16, the sinks stay fp32. These GPT-OSS-shaped tensors stand in for a serving
# engine's KV cache during RL rollouts; no dataset or weight is used.

DECODE_WORKLOADS = {
    # name: (B, Lk range, Nq, Hq, Hkv, window)
    "decode32k": (8, (16384, 32768), 1, 64, 8, 0),
    "decode32k_nq4": (8, (16384, 32768), 4, 64, 8, 0),
    "decode32k_window": (8, (16384, 32768), 1, 64, 8, 128),
}


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [Tq, Hq, d] bf16 (CPU): the new tokens' queries
    k: torch.Tensor            # [Tk, Hkv, d] bf16: the caches (new tokens included)
    v: torch.Tensor
    sinks: torch.Tensor        # [Hq] fp32
    cu_q: torch.Tensor         # [B+1] int32
    cu_k: torch.Tensor         # [B+1] int32
    max_q: int
    max_k: int
    window: int


def make_decode_inputs(lengths_k, nq, hq: int, hkv: int, d: int = 64, window: int = 0, seed: int = 0,
                       sink_scale: float = 1.0) -> DecodeInputs:
    lengths_k = tuple(int(x) for x in lengths_k)
    nqs = [int(nq)] * len(lengths_k) if isinstance(nq, int) else [int(x) for x in nq]
    nqs = tuple(min(a, b) for a, b in zip(nqs, lengths_k))  # a sequence has at most Lk new tokens
    Tk, Tq = sum(lengths_k), sum(nqs)
    gen = torch.Generator().manual_seed(seed)
    k = torch.randn((Tk, hkv, d), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((Tk, hkv, d), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((Tq, hq, d), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    sinks = torch.randn((hq,), generator=gen, dtype=torch.float32) * sink_scale
    return DecodeInputs(q, k, v, sinks, cu_from_lengths(nqs), cu_from_lengths(lengths_k), max(nqs, default=0),
                        max(lengths_k, default=0), int(window))


def make_decode_workload_inputs(name: str, seed: int = 0) -> DecodeInputs:
    B, (lo, hi), nq, hq, hkv, window = DECODE_WORKLOADS[name]
    lengths = np.random.default_rng(seed).integers(lo, hi, B, endpoint=True)
    return make_decode_inputs(lengths, nq, hq, hkv, 64, window, seed)


def last_rows(cu_seqlens, nq):
    """Row indices of the last nq[b] tokens of every packed sequence, and their offsets [B+1]."""
    cu = [int(x) for x in cu_seqlens]
    rows, cu_q = [], [0]
    for b in range(len(cu) - 1):
        n = min(int(nq[b]), cu[b + 1] - cu[b])
        rows += list(range(cu[b + 1] - n, cu[b + 1]))
        cu_q.append(cu_q[-1] + n)
    return rows, torch.tensor(cu_q, dtype=torch.int32)
