"""Pins for the fp64 oracle against facts the pages and the mathematics fix (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped sink term, a scaled sink, a
wrong sign in dL/dS_h, a transposed operand, an off-by-one window) fails at least one of them;
``test_planted_mistakes_are_caught`` plants such slips in the oracle and checks exactly that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sink_attention as sa
from workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def f64(t):
    return t.detach().to(torch.float64).numpy()


def _small(lengths=(37, 0, 1, 60), hq=4, hkv=2, d=16, causal=True, window=0, seed=3, **kw):
    return make_inputs(lengths, hq, hkv, d, causal=causal, window=window, seed=seed, **kw)


# ---------------------------------------------------------------------------------------------
# Golden: hand-worked values (tests/golden/hand_worked.json)
# ---------------------------------------------------------------------------------------------

def _val(x):
    if isinstance(x, list) and len(x) == 2 and all(isinstance(y, int) for y in x):
        return x[0] / x[1]
    if isinstance(x, str):
        return {"ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4), "1+ln2": 1 + math.log(2)}[x]
    return float(x)


def _arr(nested):
    if isinstance(nested, list) and not (len(nested) == 2 and all(isinstance(y, int) for y in nested)):
        return np.array([_arr(x) for x in nested])
    return _val(nested)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_golden_hand_worked(case):
    q = np.array(case["q"], dtype=float)
    k = np.array(case["k"], dtype=float)
    v = np.array(case["v"], dtype=float)
    dout = np.array(case["dout"], dtype=float)
    sinks = np.array([_val(s) for s in case["sinks"]])
    cu = np.concatenate([[0], np.cumsum(case["lengths"])])
    kw = dict(causal=case["causal"], window=case["window"], scale=case["scale"])
    ex = case["expect"]
    out, lse = oracle.forward(q, k, v, sinks, cu, **kw)
    np.testing.assert_allclose(out, _arr(ex["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, _arr(ex["lse"]), rtol=0, atol=1e-14)
    _, ps = oracle.probabilities(q, k, sinks, cu, **kw)
    np.testing.assert_allclose(ps, _arr(ex["p_sink"]), rtol=0, atol=1e-14)
    if "dq" in ex:
        dq, dk, dv, ds = oracle.backward(q, k, v, sinks, dout, cu, **kw)
        np.testing.assert_allclose(dq, _arr(ex["dq"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dk, _arr(ex["dk"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dv, _arr(ex["dv"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(ds, _arr(ex["dsinks"]), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------------------------
# Special case S_h -> -inf reduces to plain softmax attention (a library routine)
# ---------------------------------------------------------------------------------------------

def _sdpa_reference(inp, scale=None):
    """Torch fp64 scaled_dot_product_attention per sequence with an explicit boolean mask."""
    hq, hkv = inp.q.shape[1], inp.k.shape[1]
    G = hq // hkv
    q = inp.q.double().requires_grad_(True)
    k = inp.k.double().requires_grad_(True)
    v = inp.v.double().requires_grad_(True)
    cu = inp.cu_seqlens.tolist()
    outs, lses = [], []
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        L = e - a
        if L == 0:
            continue
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        mask = torch.ones(L, L, dtype=torch.bool)
        if inp.causal:
            mask &= j <= i
        if inp.window > 0:
            mask &= j > i - inp.window
            if not inp.causal:
                mask &= j < i + inp.window
        qs = q[a:e].transpose(0, 1)                                   # [H, L, d]
        ks = k[a:e].repeat_interleave(G, dim=1).transpose(0, 1)
        vs = v[a:e].repeat_interleave(G, dim=1).transpose(0, 1)
        o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, scale=scale)
        outs.append(o.transpose(0, 1))
        sc = (qs @ ks.transpose(1, 2)) * (scale if scale else 1 / math.sqrt(q.shape[-1]))
        lses.append(torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=-1))
    out = torch.cat(outs, 0)
    out.backward(inp.dout.double())
    return out.detach().numpy(), torch.cat(lses, 1).detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 5), (False, 0), (False, 5)])
@pytest.mark.parametrize("hkv", [1, 2, 4])
def test_neg_inf_sink_is_plain_attention(causal, window, hkv):
    inp = _small(lengths=(23, 1, 40), hq=4, hkv=hkv, causal=causal, window=window,
                 sinks_override=[-math.inf] * 4)
    out, lse = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, causal, window)
    dq, dk, dv, ds = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, causal, window)
    ro, rl, rdq, rdk, rdv = _sdpa_reference(inp)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, rdq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, rdk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, rdv, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(ds, np.zeros(4))


def test_neg_inf_sink_non_default_scale():
    inp = _small(lengths=(19, 30), hq=2, hkv=1, sinks_override=[-math.inf] * 2)
    out, lse = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, True, 0, scale=0.3)
    ro, rl, *_ = _sdpa_reference(inp, scale=0.3)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# Normalisation invariant: sum_j P_ij + P_sink = 1
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", [(True, 0), (True, 7), (False, 0), (False, 7)])
def test_probabilities_sum_to_one(causal, window):
    inp = _small(lengths=(50,), hq=3, hkv=1, causal=causal, window=window, sink_scale=3.0)
    P, Ps = oracle.probabilities(inp.q, inp.k, inp.sinks, inp.cu_seqlens, causal, window)
    np.testing.assert_allclose(P.sum(-1) + Ps, 1.0, rtol=0, atol=1e-14)
    assert (Ps > 0).all() and (P >= 0).all()
    # LSE is the log of the full denominator: P_sink = exp(S_h - LSE)
    _, lse = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, causal, window)
    np.testing.assert_allclose(Ps, np.exp(f64(inp.sinks)[:, None] - lse), rtol=1e-13)


# ---------------------------------------------------------------------------------------------
# Closed forms: uniform scores (Q = 0) and row-constant scores (all K_j equal)
# ---------------------------------------------------------------------------------------------

def _n_visible(L, causal, window):
    i = np.arange(L)
    if not causal:
        if window > 0:  # keys i - W < j < i + W inside [0, L)
            return np.minimum(i + window, L) - np.maximum(i - window + 1, 0)
        return np.full(L, L)
    return np.minimum(i + 1, window) if window > 0 else i + 1


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 4), (False, 0), (False, 4)])
def test_uniform_scores_closed_form(causal, window):
    L = 29
    inp = _small(lengths=(L,), hq=2, hkv=1, causal=causal, window=window, zero_q=True)
    sinks = f64(inp.sinks)
    out, lse = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, causal, window)
    dq, dk, dv, ds = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, causal, window)
    n = _n_visible(L, causal, window)
    V = f64(inp.v)[:, 0]
    dO = f64(inp.dout)
    for h in range(2):
        denom = n + np.exp(sinks[h])                                   # P_ij = 1/(n_i + e^{S_h})
        np.testing.assert_allclose(lse[h], np.log(denom), rtol=0, atol=1e-13)
        for i in range(L):
            js = [j for j in range(L) if sa.visible(i, j, causal, window)]
            np.testing.assert_allclose(out[i, h], V[js].sum(0) / denom[i], rtol=0, atol=1e-13)
    # dV_j = sum over rows i that see j, over heads, of dO_i / (n_i + e^{S_h})
    for j in range(L):
        acc = np.zeros(V.shape[1])
        for h in range(2):
            denom = n + np.exp(sinks[h])
            for i in range(L):
                if sa.visible(i, j, causal, window):
                    acc += dO[i, h] / denom[i]
        np.testing.assert_allclose(dv[j, 0], acc, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)                  # dK = scale dS^T Q = 0


def test_row_constant_scores_closed_form():
    """All keys equal => S_ij = s_i for every visible j: P_ij = 1/(n_i + e^{S_h - s_i})."""
    L = 21
    inp = _small(lengths=(L,), hq=1, hkv=1, d=8)
    k = inp.k.clone()
    k[:] = k[0:1]
    s = f64(inp.q)[:, 0] @ f64(k)[0, 0] / math.sqrt(8)
    sink = float(inp.sinks[0])
    out, lse = oracle.forward(inp.q, k, inp.v, inp.sinks, inp.cu_seqlens, True, 0)
    n = np.arange(1, L + 1)
    np.testing.assert_allclose(lse[0], s + np.log(n + np.exp(sink - s)), rtol=0, atol=1e-13)
    V = f64(inp.v)[:, 0]
    expect = np.cumsum(V, axis=0) / (n + np.exp(sink - s))[:, None]
    np.testing.assert_allclose(out[:, 0], expect, rtol=0, atol=1e-13)


def test_single_key_is_logistic():
    inp = _small(lengths=(1, 1, 1), hq=2, hkv=1, d=8, sink_scale=2.0)
    P, Ps = oracle.probabilities(inp.q, inp.k, inp.sinks, inp.cu_seqlens, True, 0, seq=1)
    q = f64(inp.q)[1]
    kk = f64(inp.k)[1, 0]
    for h in range(2):
        s00 = q[h] @ kk / math.sqrt(8)
        sig = 1 / (1 + math.exp(-(s00 - float(inp.sinks[h]))))
        assert abs(P[h, 0, 0] - sig) < 1e-15
        assert abs(Ps[h, 0] - (1 - sig)) < 1e-15


# ---------------------------------------------------------------------------------------------
# Finite differences of L = sum(dout * O) for every input, sinks included
# ---------------------------------------------------------------------------------------------

def _loss(q, k, v, s, cu, dout, causal, window):
    out, _ = oracle.forward(q, k, v, s, cu, causal, window)
    return float((out * dout).sum())


@pytest.mark.parametrize("lengths,causal,window", [((3, 5), True, 0), ((3, 5), True, 2), ((4, 0, 4), False, 0),
                                                    ((1, 6), True, 3), ((4, 6), False, 2)])
def test_finite_differences(lengths, causal, window):
    inp = _small(lengths=lengths, hq=2, hkv=1, d=4, causal=causal, window=window, seed=11)
    q, k, v, s, dout = f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.sinks), f64(inp.dout)
    cu = inp.cu_seqlens.numpy()
    dq, dk, dv, ds = oracle.backward(q, k, v, s, dout, cu, causal, window)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("s", s, ds)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v, "s": s}
            plus = {n: a.copy() for n, a in args.items()}
            minus = {n: a.copy() for n, a in args.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            num[idx] = (_loss(plus["q"], plus["k"], plus["v"], plus["s"], cu, dout, causal, window)
                        - _loss(minus["q"], minus["k"], minus["v"], minus["s"], cu, dout, causal, window)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)


# ---------------------------------------------------------------------------------------------
# Independent route: torch fp64 autograd of the pages' pseudocode (concat / softmax / slice / @)
# ---------------------------------------------------------------------------------------------

def _pseudocode_autograd(inp):
    hq, hkv = inp.q.shape[1], inp.k.shape[1]
    G = hq // hkv
    q = inp.q.double().requires_grad_(True)
    k = inp.k.double().requires_grad_(True)
    v = inp.v.double().requires_grad_(True)
    sink = inp.sinks.double().requires_grad_(True)
    d = q.shape[-1]
    outs = []
    cu = inp.cu_seqlens.tolist()
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        L = e - a
        if L == 0:
            continue
        Q = q[a:e].transpose(0, 1)
        K = k[a:e].repeat_interleave(G, 1).transpose(0, 1)
        V = v[a:e].repeat_interleave(G, 1).transpose(0, 1)
        scores = Q @ K.transpose(1, 2) / math.sqrt(d)                  # [H, N_q, N_k]
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        keep = torch.ones(L, L, dtype=torch.bool)
        if inp.causal:
            keep &= j <= i
        if inp.window > 0:
            keep &= j > i - inp.window
            if not inp.causal:
                keep &= j < i + inp.window
        scores = scores.masked_fill(~keep, -math.inf)
        combined = torch.cat([scores, sink[:, None, None].expand(hq, L, 1)], dim=-1)
        probs = torch.softmax(combined, dim=-1)
        probs_content = probs[..., :-1]
        outs.append((probs_content @ V).transpose(0, 1))
    out = torch.cat(outs, 0)
    out.backward(inp.dout.double())
    return out.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), sink.grad.numpy()


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 16), (False, 0), (False, 16)])
def test_matches_autograd_of_pseudocode(causal, window):
    inp = make_inputs((256,), 4, 2, 64, causal=causal, window=window, seed=5)
    out, _ = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, causal, window, row_block=100)
    dq, dk, dv, ds = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, causal, window,
                                     row_block=100)
    ro, rdq, rdk, rdv, rds = _pseudocode_autograd(inp)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(dq, rdq, atol=1e-11)
    np.testing.assert_allclose(dk, rdk, atol=1e-11)
    np.testing.assert_allclose(dv, rdv, atol=1e-11)
    np.testing.assert_allclose(ds, rds, rtol=1e-10, atol=1e-11)


def test_varlen_autograd_of_pseudocode():
    inp = make_inputs((37, 0, 1, 90), 4, 1, 32, causal=True, window=0, seed=9, sink_scale=3.0)
    dq, dk, dv, ds = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, True, 0)
    _, rdq, rdk, rdv, rds = _pseudocode_autograd(inp)
    np.testing.assert_allclose(dq, rdq, atol=1e-11)
    np.testing.assert_allclose(dk, rdk, atol=1e-11)
    np.testing.assert_allclose(dv, rdv, atol=1e-11)
    np.testing.assert_allclose(ds, rds, rtol=1e-10, atol=1e-11)


# ---------------------------------------------------------------------------------------------
# Identities
# ---------------------------------------------------------------------------------------------

def test_identities_D_and_shift_invariance():
    inp = _small(lengths=(45,), hq=2, hkv=1, d=16, window=0)
    q, k, v, dout = f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.dout)
    P, Ps = oracle.probabilities(q, k, inp.sinks, inp.cu_seqlens, True, 0)
    out, _ = oracle.forward(q, k, v, inp.sinks, inp.cu_seqlens, True, 0)
    _, _, _, ds = oracle.backward(q, k, v, inp.sinks, dout, inp.cu_seqlens, True, 0)
    for h in range(2):
        dP = dout[:, h] @ v[:, 0].T
        D_tilde = (P[h] * dP).sum(1)
        D = (dout[:, h] * out[:, h]).sum(1)                            # rowsum(dO * O)
        np.testing.assert_allclose(D, D_tilde, rtol=1e-12, atol=1e-14)
        dS = P[h] * (dP - D[:, None])
        # softmax shift invariance: each combined row's gradient sums to zero
        np.testing.assert_allclose(dS.sum() + ds[h], 0.0, atol=1e-12)
        np.testing.assert_allclose(ds[h], -(Ps[h] * D).sum(), rtol=1e-12)


# ---------------------------------------------------------------------------------------------
# Plumbing reductions: GQA == MHA on repeated K/V, varlen == concatenated runs, W >= L == causal
# ---------------------------------------------------------------------------------------------

def test_gqa_equals_repeated_mha():
    inp = _small(lengths=(33, 20), hq=8, hkv=2, d=16)
    G = 4
    kr = inp.k.repeat_interleave(G, dim=1)
    vr = inp.v.repeat_interleave(G, dim=1)
    o1, l1 = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, True, 0)
    o2, l2 = oracle.forward(inp.q, kr, vr, inp.sinks, inp.cu_seqlens, True, 0)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    g1 = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, True, 0)
    g2 = oracle.backward(inp.q, kr, vr, inp.sinks, inp.dout, inp.cu_seqlens, True, 0)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-13)
    np.testing.assert_allclose(g1[1], g2[1].reshape(g2[1].shape[0], 2, G, -1).sum(2), atol=1e-12)
    np.testing.assert_allclose(g1[2], g2[2].reshape(g2[2].shape[0], 2, G, -1).sum(2), atol=1e-12)
    np.testing.assert_allclose(g1[3], g2[3], atol=1e-13)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 6), (False, 0), (False, 6)])
def test_varlen_equals_concatenated_runs(causal, window):
    lengths = (17, 0, 1, 40, 9)
    inp = _small(lengths=lengths, hq=4, hkv=2, d=8, causal=causal, window=window)
    o, l = oracle.forward(inp.q, inp.k, inp.v, inp.sinks, inp.cu_seqlens, causal, window)
    dq, dk, dv, ds = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, causal, window)
    cu = inp.cu_seqlens.tolist()
    ds_sum = np.zeros(4)
    for b in range(len(lengths)):
        a, e = cu[b], cu[b + 1]
        one = torch.tensor([0, e - a], dtype=torch.int32)
        ob, lb = oracle.forward(inp.q[a:e], inp.k[a:e], inp.v[a:e], inp.sinks, one, causal, window)
        gb = oracle.backward(inp.q[a:e], inp.k[a:e], inp.v[a:e], inp.sinks, inp.dout[a:e], one, causal, window)
        np.testing.assert_allclose(o[a:e], ob, atol=1e-14)
        np.testing.assert_allclose(l[:, a:e], lb, atol=1e-14)
        np.testing.assert_allclose(dq[a:e], gb[0], atol=1e-14)
        np.testing.assert_allclose(dk[a:e], gb[1], atol=1e-14)
        np.testing.assert_allclose(dv[a:e], gb[2], atol=1e-14)
        ds_sum += gb[3]
    np.testing.assert_allclose(ds, ds_sum, atol=1e-13)


def test_window_at_least_length_is_causal():
    inp = _small(lengths=(30, 12), hq=2, hkv=1, d=8)
    a = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, True, 0, return_forward=True)
    b = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, True, 30, return_forward=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_window_boundary_pair():
    """Window W: key i-W is excluded, key i-W+1 is included (exactly W keys incl. itself)."""
    W = 3
    inp = _small(lengths=(12,), hq=1, hkv=1, d=8, window=W)
    P, _ = oracle.probabilities(inp.q, inp.k, inp.sinks, inp.cu_seqlens, True, W)
    for i in range(W, 12):
        assert P[0, i, i - W] == 0.0
        assert P[0, i, i - W + 1] > 0.0
        assert (P[0, i] > 0).sum() == W


def test_symmetric_window_boundary_pairs():
    """Non-causal window W: keys i-W and i+W are excluded, keys i-W+1 and i+W-1 included."""
    W, L = 3, 12
    inp = _small(lengths=(L,), hq=1, hkv=1, d=8, causal=False, window=W)
    P, _ = oracle.probabilities(inp.q, inp.k, inp.sinks, inp.cu_seqlens, False, W)
    for i in range(L):
        if i - W >= 0:
            assert P[0, i, i - W] == 0.0
        if i + W < L:
            assert P[0, i, i + W] == 0.0
        assert P[0, i, max(i - W + 1, 0)] > 0.0 and P[0, i, min(i + W - 1, L - 1)] > 0.0
        assert (P[0, i] > 0).sum() == min(i + W, L) - max(i - W + 1, 0)


def test_symmetric_window_at_least_length_is_full():
    inp = _small(lengths=(30, 12), hq=2, hkv=1, d=8, causal=False)
    a = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, False, 0, return_forward=True)
    b = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, False, 30, return_forward=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_row_block_does_not_change_results():
    inp = _small(lengths=(70,), hq=2, hkv=1, d=16, window=9)
    a = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, True, 9, return_forward=True)
    b = oracle.backward(inp.q, inp.k, inp.v, inp.sinks, inp.dout, inp.cu_seqlens, True, 9, row_block=7,
                        return_forward=True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# Row-sampled helpers (used for full-size checks) agree with the full oracle
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", [(True, 0), (True, 5), (False, 0), (False, 5)])
def test_sampled_helpers_agree_with_full(causal, window):
    inp = _small(lengths=(26, 1, 31), hq=4, hkv=2, d=16, causal=causal, window=window)
    args = (inp.q, inp.k, inp.v, inp.sinks)
    out, lse = oracle.forward(*args, inp.cu_seqlens, causal, window)
    dq, dk, dv, ds = oracle.backward(*args, inp.dout, inp.cu_seqlens, causal, window)
    rows = [0, 5, 25, 26, 27, 57]
    heads = [0, 3]
    o_s, l_s = oracle.forward_rows(*args, inp.cu_seqlens, rows, heads, causal=causal, window=window)
    np.testing.assert_allclose(o_s, out[rows][:, heads], atol=1e-14)
    np.testing.assert_allclose(l_s, lse[heads][:, rows], atol=1e-14)
    dq_s = oracle.dq_rows(*args, inp.dout, inp.cu_seqlens, rows, heads, causal=causal, window=window)
    np.testing.assert_allclose(dq_s, dq[rows][:, heads], atol=1e-14)
    keys = [0, 3, 25, 26, 30, 57]
    dk_s, dv_s = oracle.dkdv_keys(*args, inp.dout, inp.cu_seqlens, keys, [0, 1], causal=causal, window=window,
                                  row_block=4)
    np.testing.assert_allclose(dk_s, dk[keys], atol=1e-13)
    np.testing.assert_allclose(dv_s, dv[keys], atol=1e-13)
    ds_s = oracle.dsink_heads(*args, inp.dout, inp.cu_seqlens, [1, 2], causal=causal, window=window)
    np.testing.assert_allclose(ds_s, ds[[1, 2]], atol=1e-13)


def test_row_without_visible_key():
    """Degenerate reading: a row that sees no key has P_sink = 1, O = 0, LSE = S_h."""
    q = np.zeros((1, 1, 2))
    k = np.ones((1, 1, 2))
    v = np.ones((1, 1, 2))
    sinks = np.array([0.7])
    c0, c1, probs, lse = sa._combined_softmax(q[:, 0], k[:, 0], np.array([0]), 1, 0.7, True, 0, 1.0)
    # window 0 and causal: the row sees key 0; force a row with none by a zero-width key range
    cols_none = sa._combined_softmax(q[:, 0], k[:0, 0], np.array([0]), 0, 0.7, True, 0, 1.0)
    _, _, p_none, lse_none = cols_none
    assert p_none.shape == (1, 1) and p_none[0, 0] == 1.0 and lse_none[0] == 0.7
    _, _, p_inf, lse_inf = sa._combined_softmax(q[:, 0], k[:0, 0], np.array([0]), 0, -np.inf, True, 0, 1.0)
    assert p_inf[0, 0] == 0.0 and lse_inf[0] == -np.inf
    assert probs.shape == (1, 2) and abs(probs.sum() - 1) < 1e-15 and c1 - c0 == 1


# ---------------------------------------------------------------------------------------------
# Planted mistakes: the pins above must catch plausible slips in the oracle
# ---------------------------------------------------------------------------------------------

def _scaled_sink_softmax(q_rows, Kg, rows, L, sink, causal, window, scale):
    return _ORIG_SOFTMAX(q_rows, Kg, rows, L, sink * scale, causal, window, scale)


def _no_sink_softmax(q_rows, Kg, rows, L, sink, causal, window, scale):
    return _ORIG_SOFTMAX(q_rows, Kg, rows, L, -np.inf, causal, window, scale)


def _off_by_one_window(q_rows, Kg, rows, L, sink, causal, window, scale):
    return _ORIG_SOFTMAX(q_rows, Kg, rows, L, sink, causal, window + 1 if window else 0, scale)


def _one_sided_window(q_rows, Kg, rows, L, sink, causal, window, scale):
    # treats a non-causal window like a causal one on the right-hand side (keys j <= i only)
    return _ORIG_SOFTMAX(q_rows, Kg, rows, L, sink, causal or window > 0, window, scale)


def _flipped_sink_grad(probs, dout_rows, Vcols):
    dS, dsink, D = _ORIG_GRADS(probs, dout_rows, Vcols)
    return dS, -dsink, D


def _dropped_D(probs, dout_rows, Vcols):
    dP = dout_rows @ Vcols.T
    g = np.concatenate([dP, np.zeros((dP.shape[0], 1))], axis=1)
    dcomb = probs * g
    return dcomb[:, :-1], dcomb[:, -1], None


_ORIG_SOFTMAX = sa._combined_softmax
_ORIG_GRADS = sa._prob_grads


def _pins_pass():
    """Run a compact subset of the pins; return False as soon as one fails."""
    checks = [lambda: test_golden_hand_worked(json.load(open(GOLDEN))["cases"][0]),
              lambda: test_golden_hand_worked(json.load(open(GOLDEN))["cases"][2]),
              lambda: test_uniform_scores_closed_form(True, 4),
              lambda: test_probabilities_sum_to_one(True, 7),
              lambda: test_finite_differences((3, 5), True, 2),
              lambda: test_window_boundary_pair(),
              lambda: test_symmetric_window_boundary_pairs()]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


@pytest.mark.parametrize("mutant", ["scaled_sink", "no_sink", "window_off_by_one", "one_sided_window",
                                     "flipped_sink_grad", "dropped_D"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    assert _pins_pass(), "pins must pass on the unmodified oracle"
    if mutant == "scaled_sink":
        monkeypatch.setattr(sa, "_combined_softmax", _scaled_sink_softmax)
    elif mutant == "no_sink":
        monkeypatch.setattr(sa, "_combined_softmax", _no_sink_softmax)
    elif mutant == "window_off_by_one":
        monkeypatch.setattr(sa, "_combined_softmax", _off_by_one_window)
    elif mutant == "one_sided_window":
        monkeypatch.setattr(sa, "_combined_softmax", _one_sided_window)
    elif mutant == "flipped_sink_grad":
        monkeypatch.setattr(sa, "_prob_grads", _flipped_sink_grad)
    elif mutant == "dropped_D":
        monkeypatch.setattr(sa, "_prob_grads", _dropped_D)
    assert not _pins_pass(), f"planted mistake {mutant} went unnoticed"
