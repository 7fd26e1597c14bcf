"""Plain, slow, fp64 CPU oracle for scaled dot-product attention with a learnable per-head sink.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product path. It shares no code with the HIP
library or its binding. Everything is NumPy float64; inputs are upcast exactly from the bf16 /
fp32 tensors the GPU receives.

What it computes, and where the pages define it
-----------------------------------------------
Pages: [nmedialink] "惊爆！GPT-OSS-20B强化学习，训练速度狂飙、超稳定！" (nmedialink.com);
[dailytechsnack] "GPT-OSS lernt stabile Werkzeugnutzung durch Agentic RL" (dailytechsnack.ch).

* Scores: S_ij = scale * Q_i . K_j with scale = 1/sqrt(d) by default
  ([nmedialink] section "标准注意力机制回顾" (standard attention recap), first pseudocode line;
  section "数学公式深入解读" (formulas), definition of S_ij).
* Sink: one learnable logit S_h per (query) head, a virtual token that is appended to each row of
  scores as one extra column, softmaxed with them, then dropped before multiplying by V
  ([nmedialink] section "GPT-OSS中的带注意力槽的注意力机制" (attention with sinks), pseudocode
  concat / softmax / slice / matmul; section "FlashAttentionV3对注意力槽的支持" (one scalar per
  head acting as a virtual token); [dailytechsnack] section "Attention Sinks brauchten einen
  vollständigen Kernel").
* P_ij = exp(S_ij) / (sum_j' exp(S_ij') + exp(S_h)) and the sink probability
  P_{i,h} = exp(S_h) / (same denominator) ([nmedialink] "数学公式深入解读", eq. for P_ij and
  eq. for P_{i,h}).
* Backward: the softmax over the combined row (content scores plus the sink column) is
  differentiated by its Jacobian. The upstream gradient with respect to a content probability is
  dP_ij = dO_i . V_j; the sink column has no value row, so its upstream gradient is 0. This gives
  dS_ij = P_ij (dP_ij - D_i) with D_i = sum_j P_ij dP_ij, and the sink column's gradient
  P_{i,h} (0 - D_i), whose sum over rows is dL/dS_h = -sum_i P_{i,h} sum_j P_ij dP_ij
  ([nmedialink] section "反向传播的实现" (backward), the simplified equation after setting the
  sink's own score gradient to zero). The printed general form in that section is garbled (it
  writes dL/dS where the upstream probability gradient is meant and flips the outer sign); the
  simplified equation is the one followed, read with "dL/dS_ij" as dL/dP_ij.
* dQ_i = scale sum_j dS_ij K_j, dK_j = scale sum_i dS_ij Q_i, dV_j = sum_i P_ij dO_i (chain rule
  through S = scale Q K^T and O = P V; the pages only state that a backward exists).

Readings where the pages are silent (each listed in the design notes):
* The sink is added after scaling (it is concatenated to the already scaled scores) and is never
  masked by causality or the window; it does not count toward the window.
* Sliding window W > 0: query i sees keys j with i - W < j <= i (exactly W keys including
  itself). Causal: j <= i. The sink is visible from every row.
* Non-causal with a window W > 0 (the pages only train with causal windows; this is the plain
  symmetric reading): query i sees keys j with |i - j| < W, i.e. i - W < j < i + W.
* GQA: query head h reads KV head h // (Hq / Hkv). Sinks are per query head.
* Varlen: sequences are packed back to back; cu_seqlens[b] .. cu_seqlens[b+1] are the rows of
  sequence b, and attention never crosses a sequence boundary ([nmedialink] section
  "结合Flash Attention V3的序列并行技术" (sequence parallelism), packed token list).
* LSE_i = log(sum_visible exp(S_ij) + exp(S_h)), natural log, including the sink.
* dL/dS_h sums over every row of every packed sequence (one shared parameter per head).
* A row with no visible key has P_sink = 1, O = 0, LSE = S_h; if the sink is also -inf its
  probabilities are all 0 and LSE = -inf.

Row blocking bounds memory only; every row's arithmetic is the plain definition above.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = ["forward", "backward", "probabilities", "forward_rows", "dq_rows", "dkdv_keys",
           "dsink_heads", "visible"]


def _f64(x) -> np.ndarray:
    """Exact upcast to float64 (torch bf16/fp32 tensors or array-likes)."""
    if hasattr(x, "detach"):
        import torch  # only for the conversion of caller-provided tensors
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def visible(i, j, causal: bool, window: int) -> np.ndarray:
    """Whether query i may attend to key j of the same sequence (the sink is always visible)."""
    i = np.asarray(i)
    j = np.asarray(j)
    ok = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if causal:
        ok &= j <= i
    if window is not None and window > 0:
        ok &= j > i - window
        if not causal:
            ok &= j < i + window
    return ok


def _default_scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)


def _key_range(r_lo: int, r_hi: int, L: int, causal: bool, window: int):
    """Smallest key interval [c0, c1) containing every key visible from rows r_lo..r_hi.
    Keys outside it are masked for all these rows, so they contribute exactly zero."""
    c0 = max(0, r_lo - window + 1) if window and window > 0 else 0
    if causal:
        c1 = min(L, r_hi + 1)
    else:
        c1 = min(L, r_hi + window) if window and window > 0 else L
    return c0, max(c0, c1)


def _combined_softmax(q_rows, Kg, rows, L, sink, causal, window, scale):
    """Softmax over [scores | sink] for the given local rows of one sequence and one head.

    Returns (c0, c1, probs[R, (c1-c0)+1], lse[R]); the last probs column is the sink's."""
    rows = np.asarray(rows, dtype=np.int64)
    c0, c1 = _key_range(int(rows.min()), int(rows.max()), L, causal, window)
    cols = np.arange(c0, c1)
    scores = scale * (q_rows @ Kg[c0:c1].T)
    scores = np.where(visible(rows[:, None], cols[None, :], causal, window), scores, -np.inf)
    combined = np.concatenate([scores, np.full((len(rows), 1), float(sink))], axis=1)
    m = combined.max(axis=1)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(combined - m[:, None])
    Z = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        probs = np.where(Z[:, None] > 0, e / Z[:, None], 0.0)
        lse = np.where(Z > 0, m + np.log(Z), -np.inf)
    return c0, c1, probs, lse


def _prob_grads(probs, dout_rows, Vcols):
    """Softmax-Jacobian backward over the combined row.

    dP_ij = dO_i . V_j is the upstream gradient of each content probability; the sink column
    carries none (it has no value row). Returns (dS[R, C], dsink_col[R], D[R])."""
    dP = dout_rows @ Vcols.T
    g = np.concatenate([dP, np.zeros((dP.shape[0], 1))], axis=1)
    D = (probs * g).sum(axis=1)
    dcomb = probs * (g - D[:, None])
    return dcomb[:, :-1], dcomb[:, -1], D


def _unpack(q, k, v, sinks, cu_seqlens):
    q = _f64(q)
    k = _f64(k)
    v = _f64(v) if v is not None else None
    sinks = _f64(sinks).reshape(-1)
    cu = _i64(cu_seqlens).reshape(-1)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    assert sinks.shape == (Hq,)
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    return q, k, v, sinks, cu, T, Hq, Hkv, d


def forward(q, k, v, sinks, cu_seqlens, causal: bool = True, window: int = 0,
            scale: Optional[float] = None, row_block: int = 1024):
    """O [T, Hq, d] and LSE [Hq, T] (natural log, sink included), both float64."""
    q, k, v, sinks, cu, T, Hq, Hkv, d = _unpack(q, k, v, sinks, cu_seqlens)
    scale = _default_scale(d, scale)
    G = Hq // Hkv
    out = np.zeros((T, Hq, d))
    lse = np.full((Hq, T), -np.inf)
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        L = e - a
        if L == 0:
            continue
        for h in range(Hq):
            Kg, Vg = k[a:e, h // G], v[a:e, h // G]
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                rows = np.arange(r0, r1)
                c0, c1, probs, lse_r = _combined_softmax(q[a + r0:a + r1, h], Kg, rows, L, sinks[h],
                                                         causal, window, scale)
                out[a + r0:a + r1, h] = probs[:, :-1] @ Vg[c0:c1]
                lse[h, a + r0:a + r1] = lse_r
    return out, lse


def backward(q, k, v, sinks, dout, cu_seqlens, causal: bool = True, window: int = 0,
             scale: Optional[float] = None, row_block: int = 1024, return_forward: bool = False):
    """dQ [T, Hq, d], dK [T, Hkv, d], dV [T, Hkv, d], dSink [Hq] (float64) of L = sum(dout * O)."""
    q, k, v, sinks, cu, T, Hq, Hkv, d = _unpack(q, k, v, sinks, cu_seqlens)
    dout = _f64(dout)
    scale = _default_scale(d, scale)
    G = Hq // Hkv
    dq = np.zeros((T, Hq, d))
    dk = np.zeros((T, Hkv, d))
    dv = np.zeros((T, Hkv, d))
    dsinks = np.zeros(Hq)
    out = np.zeros((T, Hq, d)) if return_forward else None
    lse = np.full((Hq, T), -np.inf) if return_forward else None
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        L = e - a
        if L == 0:
            continue
        for h in range(Hq):
            g = h // G
            Kg, Vg = k[a:e, g], v[a:e, g]
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                rows = np.arange(r0, r1)
                q_rows = q[a + r0:a + r1, h]
                do_rows = dout[a + r0:a + r1, h]
                c0, c1, probs, lse_r = _combined_softmax(q_rows, Kg, rows, L, sinks[h], causal, window, scale)
                dS, dsink_col, _ = _prob_grads(probs, do_rows, Vg[c0:c1])
                dq[a + r0:a + r1, h] = scale * (dS @ Kg[c0:c1])
                dk[a + c0:a + c1, g] += scale * (dS.T @ q_rows)
                dv[a + c0:a + c1, g] += probs[:, :-1].T @ do_rows
                dsinks[h] += dsink_col.sum()
                if return_forward:
                    out[a + r0:a + r1, h] = probs[:, :-1] @ Vg[c0:c1]
                    lse[h, a + r0:a + r1] = lse_r
    if return_forward:
        return dq, dk, dv, dsinks, out, lse
    return dq, dk, dv, dsinks


def probabilities(q, k, sinks, cu_seqlens, causal: bool = True, window: int = 0,
                  scale: Optional[float] = None, seq: int = 0):
    """Full probability matrices of one sequence (small inputs): P [Hq, L, L], P_sink [Hq, L]."""
    q, k, _, sinks, cu, T, Hq, Hkv, d = _unpack(q, k, None, sinks, cu_seqlens)
    scale = _default_scale(d, scale)
    G = Hq // Hkv
    a, e = int(cu[seq]), int(cu[seq + 1])
    L = e - a
    P = np.zeros((Hq, L, L))
    Ps = np.zeros((Hq, L))
    if L == 0:
        return P, Ps
    rows = np.arange(L)
    for h in range(Hq):
        c0, c1, probs, _ = _combined_softmax(q[a:e, h], k[a:e, h // G], rows, L, sinks[h], causal, window, scale)
        P[h, :, c0:c1] = probs[:, :-1]
        Ps[h] = probs[:, -1]
    return P, Ps


def _locate(cu, t):
    b = int(np.searchsorted(cu, t, side="right") - 1)
    return b, int(cu[b]), int(cu[b + 1])


def forward_rows(q, k, v, sinks, cu_seqlens, rows: Iterable[int], heads: Sequence[int],
                 causal: bool = True, window: int = 0, scale: Optional[float] = None):
    """O and LSE of selected packed rows (global token indices) and query heads, each row on its own:
    O [n_rows, n_heads, d], LSE [n_heads, n_rows]."""
    q, k, v, sinks, cu, T, Hq, Hkv, d = _unpack(q, k, v, sinks, cu_seqlens)
    scale = _default_scale(d, scale)
    G = Hq // Hkv
    rows = list(rows)
    out = np.zeros((len(rows), len(heads), d))
    lse = np.zeros((len(heads), len(rows)))
    for ri, t in enumerate(rows):
        b, a, e = _locate(cu, t)
        L = e - a
        i = t - a
        for hi, h in enumerate(heads):
            Kg, Vg = k[a:e, h // G], v[a:e, h // G]
            c0, c1, probs, lse_r = _combined_softmax(q[t:t + 1, h], Kg, np.array([i]), L, sinks[h],
                                                     causal, window, scale)
            out[ri, hi] = (probs[:, :-1] @ Vg[c0:c1])[0]
            lse[hi, ri] = lse_r[0]
    return out, lse


def dq_rows(q, k, v, sinks, dout, cu_seqlens, rows: Iterable[int], heads: Sequence[int],
            causal: bool = True, window: int = 0, scale: Optional[float] = None):
    """dQ of selected packed rows and heads, each row on its own: [n_rows, n_heads, d]."""
    q, k, v, sinks, cu, T, Hq, Hkv, d = _unpack(q, k, v, sinks, cu_seqlens)
    dout = _f64(dout)
    scale = _default_scale(d, scale)
    G = Hq // Hkv
    rows = list(rows)
    dq = np.zeros((len(rows), len(heads), d))
    for ri, t in enumerate(rows):
        b, a, e = _locate(cu, t)
        L = e - a
        i = t - a
        for hi, h in enumerate(heads):
            Kg, Vg = k[a:e, h // G], v[a:e, h // G]
            c0, c1, probs, _ = _combined_softmax(q[t:t + 1, h], Kg, np.array([i]), L, sinks[h],
                                                 causal, window, scale)
            dS, _, _ = _prob_grads(probs, dout[t:t + 1, h], Vg[c0:c1])
            dq[ri, hi] = scale * (dS @ Kg[c0:c1])[0]
    return dq


def dkdv_keys(q, k, v, sinks, dout, cu_seqlens, keys: Iterable[int], kv_heads: Sequence[int],
              causal: bool = True, window: int = 0, scale: Optional[float] = None, row_block: int = 1024):
    """dK, dV of selected packed key rows and KV heads: [n_keys, n_kv_heads, d] each.

    Each key needs the full softmax of every row that sees it; the cost grows with that row count
    (cheap near the end of a causal sequence, or anywhere under a window)."""
    q, k, v, sinks, cu, T, Hq, Hkv, d = _unpack(q, k, v, sinks, cu_seqlens)
    dout = _f64(dout)
    scale = _default_scale(d, scale)
    G = Hq // Hkv
    keys = list(keys)
    dk = np.zeros((len(keys), len(kv_heads), d))
    dv = np.zeros((len(keys), len(kv_heads), d))
    for ki, t in enumerate(keys):
        b, a, e = _locate(cu, t)
        L = e - a
        j = t - a
        all_rows = np.arange(L)
        seeing = all_rows[visible(all_rows, j, causal, window)]
        for gi, g in enumerate(kv_heads):
            Kg, Vg = k[a:e, g], v[a:e, g]
            for h in range(g * G, (g + 1) * G):
                for s0 in range(0, len(seeing), row_block):
                    rows = seeing[s0:s0 + row_block]
                    q_rows = q[a + rows, h]
                    do_rows = dout[a + rows, h]
                    c0, c1, probs, _ = _combined_softmax(q_rows, Kg, rows, L, sinks[h], causal, window, scale)
                    dS, _, _ = _prob_grads(probs, do_rows, Vg[c0:c1])
                    col = j - c0
                    dk[ki, gi] += scale * (dS[:, col] @ q_rows)
                    dv[ki, gi] += probs[:, col] @ do_rows
    return dk, dv


def dsink_heads(q, k, v, sinks, dout, cu_seqlens, heads: Sequence[int], causal: bool = True,
                window: int = 0, scale: Optional[float] = None, row_block: int = 1024,
                return_terms: bool = False):
    """dL/dS_h for selected heads (a full pass over every row of those heads).

    With ``return_terms`` also returns, per head, sum_i |P_{i,h} D_i| (the conditioning of the sum)."""
    q, k, v, sinks, cu, T, Hq, Hkv, d = _unpack(q, k, v, sinks, cu_seqlens)
    dout = _f64(dout)
    scale = _default_scale(d, scale)
    G = Hq // Hkv
    res = np.zeros(len(heads))
    absterms = np.zeros(len(heads))
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        L = e - a
        if L == 0:
            continue
        for hi, h in enumerate(heads):
            Kg, Vg = k[a:e, h // G], v[a:e, h // G]
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                rows = np.arange(r0, r1)
                c0, c1, probs, _ = _combined_softmax(q[a + r0:a + r1, h], Kg, rows, L, sinks[h],
                                                     causal, window, scale)
                _, dsink_col, _ = _prob_grads(probs, dout[a + r0:a + r1, h], Vg[c0:c1])
                res[hi] += dsink_col.sum()
                absterms[hi] += np.abs(dsink_col).sum()
    if return_terms:
        return res, absterms
    return res
