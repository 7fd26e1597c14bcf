"""Pins of the decode-forward oracle (oracle/decode.py), on CPU.

* Identity with the training-forward oracle: the new queries are the last tokens of their
  sequences, so their rows must equal the full causal forward's last rows. This transfers every
  pin of the training forward (SDPA with S_h = -inf, closed forms, finite differences) to the
  decode oracle, which shares no code with it.
* S_h = -inf equals torch fp64 scaled_dot_product_attention with an explicit bottom-right mask.
* Uniform scores (Q = 0): P = 1 / (n + exp(S_h)), LSE = log(n + exp(S_h)).
* A window covering the whole cache equals no window.
* A planted mistake (top-left alignment) fails the identity pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import decode as decode_mod
from workloads import make_inputs


def _decode_split(inp, nq):
    """Take the last nq[b] rows of every sequence as the new queries (q rows and their offsets)."""
    cu = inp.cu_seqlens.tolist()
    rows, cu_q = [], [0]
    for b in range(len(cu) - 1):
        n = min(nq[b], cu[b + 1] - cu[b])
        rows += list(range(cu[b + 1] - n, cu[b + 1]))
        cu_q.append(cu_q[-1] + n)
    return rows, torch.tensor(cu_q, dtype=torch.int32)


@pytest.mark.parametrize("window", [0, 5, 37])
@pytest.mark.parametrize("hkv", [1, 2])
def test_decode_equals_last_rows_of_forward(window, hkv):
    inp = make_inputs((40, 1, 17, 64), 4, hkv, 16, causal=True, window=window, seed=3)
    rows, cu_q = _decode_split(inp, [3, 1, 4, 1])
    out_full, lse_full = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, True, window)
    out, lse = oracle.decode_forward(inp.q[rows], inp.k, inp.v, inp.sinks, cu_q, inp.cu_seqlens, window)
    np.testing.assert_allclose(out, out_full[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_full[:, rows], rtol=0, atol=1e-12)


def test_neg_inf_sink_is_sdpa_bottom_right():
    inp = make_inputs((50, 9), 4, 2, 32, seed=5, sinks_override=[-math.inf] * 4)
    rows, cu_q = _decode_split(inp, [6, 9])
    out, lse = oracle.decode_forward(inp.q[rows], inp.k, inp.v, inp.sinks, cu_q, inp.cu_seqlens)
    cu, cq = inp.cu_seqlens.tolist(), cu_q.tolist()
    for b in range(2):
        qs = inp.q[rows][cq[b]:cq[b + 1]].double().transpose(0, 1)          # [Hq, nq, d]
        ks = inp.k[cu[b]:cu[b + 1]].double().repeat_interleave(2, dim=1).transpose(0, 1)
        vs = inp.v[cu[b]:cu[b + 1]].double().repeat_interleave(2, dim=1).transpose(0, 1)
        nq, lk = qs.shape[1], ks.shape[1]
        mask = torch.arange(lk)[None, :] <= (lk - nq + torch.arange(nq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask)
        np.testing.assert_allclose(out[cq[b]:cq[b + 1]], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
        s = (qs @ ks.transpose(1, 2)) / math.sqrt(32)
        ref_lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
        np.testing.assert_allclose(lse[:, cq[b]:cq[b + 1]], ref_lse.numpy(), rtol=0, atol=1e-12)


def test_uniform_scores_closed_form():
    inp = make_inputs((30,), 2, 1, 16, seed=2, zero_q=True)
    rows, cu_q = _decode_split(inp, [4])
    out, lse = oracle.decode_forward(inp.q[rows], inp.k, inp.v, inp.sinks, cu_q, inp.cu_seqlens, window=7)
    v = inp.v.double().numpy()[:, 0, :]
    for j in range(4):
        p = 26 + j                                   # position of new query j
        n = min(p + 1, 7)
        for h in range(2):
            z = n + math.exp(float(inp.sinks[h]))
            np.testing.assert_allclose(out[j, h], v[p - n + 1:p + 1].sum(0) / z, rtol=0, atol=1e-12)
            assert abs(lse[h, j] - math.log(z)) < 1e-12


def test_window_covering_cache_is_plain_causal():
    inp = make_inputs((25, 12), 4, 2, 16, seed=8)
    rows, cu_q = _decode_split(inp, [2, 3])
    a = oracle.decode_forward(inp.q[rows], inp.k, inp.v, inp.sinks, cu_q, inp.cu_seqlens, window=0)
    b = oracle.decode_forward(inp.q[rows], inp.k, inp.v, inp.sinks, cu_q, inp.cu_seqlens, window=25)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=0)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=0)


def test_planted_top_left_alignment_fails_identity(monkeypatch):
    inp = make_inputs((20, 9), 2, 1, 16, seed=4)
    rows, cu_q = _decode_split(inp, [3, 2])
    out_full, _ = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, True, 0)
    monkeypatch.setattr(decode_mod, "_positions", lambda lk, nq: np.arange(nq))  # top-left alignment
    out_bad, _ = oracle.decode_forward(inp.q[rows], inp.k, inp.v, inp.sinks, cu_q, inp.cu_seqlens)
    assert np.abs(out_bad - out_full[rows]).max() > 1e-2
