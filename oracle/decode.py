"""Plain fp64 CPU oracle of the inference-shaped (decode) forward with a learnable per-head sink.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (never by the product path); shares no code with
the HIP library, its binding, or the training-forward oracle in ``sink_attention.py`` (so that
the identity pin between the two is a real check).

Each packed sequence b has Lk_b cached keys / values (rows cu_k[b] .. cu_k[b+1]-1) and its last
Nq_b tokens as new queries (rows cu_q[b] .. cu_q[b+1]-1). New query j sits at position
Lk_b - Nq_b + j and, as in causal self-attention, sees the keys at positions <= its own (and,
with a window W > 0, only those > position - W), plus the sink. The sink is the per-head logit
S_h appended to each row's scaled scores, softmaxed with them and dropped before the product
with V (nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section
"GPT-OSS中的带注意力槽的注意力机制", pseudocode; section "数学公式深入解读", eq. P_ij).
LSE is the natural log of the full denominator, sink included.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = ["decode_forward"]


def _positions(lk: int, nq: int) -> np.ndarray:
    """Positions of the nq new queries in a sequence of lk tokens: its last nq tokens."""
    return lk - nq + np.arange(nq)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def decode_forward(q, k, v, sinks, cu_q, cu_k, window: int = 0, scale: Optional[float] = None):
    """O [Tq, Hq, d] and LSE [Hq, Tq] (float64) of the new queries against their sequences' caches."""
    q, k, v, sinks = _f64(q), _f64(k), _f64(v), _f64(sinks)
    cu_q = np.asarray(_f64(cu_q), dtype=np.int64)
    cu_k = np.asarray(_f64(cu_k), dtype=np.int64)
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if not scale else float(scale)
    out = np.zeros((Tq, Hq, d))
    lse = np.full((Hq, Tq), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        nq, lk = q1 - q0, k1 - k0
        if nq == 0:
            continue
        pos = _positions(lk, nq)
        key = np.arange(lk)
        vis = key[None, :] <= pos[:, None]            # causal
        if window > 0:
            vis &= key[None, :] > pos[:, None] - window
        for h in range(Hq):
            g = h // G
            s = scale * (q[q0:q1, h, :] @ k[k0:k1, g, :].T)       # [nq, lk]
            s = np.where(vis, s, -np.inf)
            logits = np.concatenate([s, np.full((nq, 1), sinks[h])], axis=1)
            m = logits.max(axis=1, keepdims=True)
            m_safe = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(logits - m_safe)
            z = e.sum(axis=1, keepdims=True)
            with np.errstate(invalid="ignore", divide="ignore"):
                p = np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)
                lse[h, q0:q1] = np.where(z[:, 0] > 0, m_safe[:, 0] + np.log(np.where(z[:, 0] > 0, z[:, 0], 1.0)),
                                         -np.inf)
            out[q0:q1, h, :] = p[:, :-1] @ v[k0:k1, g, :]
    return out, lse
