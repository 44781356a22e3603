"""Pins for the gradient oracle (oracle/backward.py); none of them reuses its code path.

* central finite differences of the forward oracle's loss sum(dO * o) in every element of q, k,
  v and the sink (the forward oracle is pinned on its own in test_oracle_pins.py);
* torch autograd (CPU, float64) through a dense formulation written here: masked scores with
  the sink appended as one extra column whose value vector is zero, softmax, drop that column;
* a closed form at window 1: each row sees only its own key, so its weight is the logistic
  function sigma(s_ii - s_h), and every gradient follows by hand;
* identities that hold at any size: sum q.dq = sum k.dk (the scores are bilinear in q and k),
  sum v.dv = sum dO.o (the output is linear in v), and without a sink sum_j dk_j = 0 for each
  sequence and KV head (adding one vector to every key shifts a whole row of scores);
* planted mistakes (sink dropped from the weights, sign of the sink gradient, missing scale on
  dk, wrong GQA accumulation, D taken over the raw dp) each fail at least one pin.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.backward as ob

RNG = np.random.default_rng(2024)


def inputs(B, L, Hq, Hkv, dqk, dv, with_sink=True, seed=0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, L, Hq, dqk))
    k = r.standard_normal((B, L, Hkv, dqk))
    v = r.standard_normal((B, L, Hkv, dv))
    do = r.standard_normal((B, L, Hq, dv))
    sink = r.standard_normal(Hq) if with_sink else None
    return q, k, v, do, sink


def loss(q, k, v, do, window, sink, scale):
    o, _ = oracle.prefill(q, k, v, window, sink, scale)
    return float((o * do).sum())


def fd_err(mod, window, with_sink, scale=0.41):
    """Largest |analytic - central difference| / (1 + |analytic|) over every input element."""
    q, k, v, do, sink = inputs(2, 6, 4, 2, 5, 3, with_sink, seed=window)
    dq, dk, dv, ds = mod.prefill_backward(q, k, v, do, window, sink, scale)
    eps = 1e-5
    worst = 0.0
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("sink", sink, ds)):
        if x is None:
            continue
        if g is None:
            return float("inf")
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = loss(q, k, v, do, window, sink, scale)
            x[idx] = keep - eps
            dn = loss(q, k, v, do, window, sink, scale)
            x[idx] = keep
            fd = (up - dn) / (2 * eps)
            worst = max(worst, abs(g[idx] - fd) / (1 + abs(g[idx])))
    return worst


def torch_grads(q, k, v, do, window, sink, scale):
    """Autograd through a dense float64 formulation with the sink as an extra zero-value key."""
    B, L, Hq, _ = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ts = torch.tensor(sink, requires_grad=True) if sink is not None else None
    kk = tk.repeat_interleave(G, dim=2)  # [B, L, Hq, d]
    vv = tv.repeat_interleave(G, dim=2)
    s = scale * torch.einsum("bihd,bjhd->bhij", tq, kk)
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    vis = (i - j >= 0) & (i - j < window)
    s = s.masked_fill(~vis, float("-inf"))
    if ts is not None:
        col = ts.view(1, Hq, 1, 1).expand(B, Hq, L, 1)
        p = torch.softmax(torch.cat([s, col], dim=-1), dim=-1)[..., :L]
    else:
        p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, vv)
    (o * torch.tensor(do)).sum().backward()
    return (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(),
            None if ts is None else ts.grad.numpy())


def autograd_err(mod, window, with_sink, scale=0.29):
    q, k, v, do, sink = inputs(2, 70, 8, 2, 12, 7, with_sink, seed=100 + window)
    got = mod.prefill_backward(q, k, v, do, window, sink, scale, block=32)
    ref = torch_grads(q, k, v, do, window, sink, scale)
    worst = 0.0
    for a, b in zip(got, ref):
        if (a is None) != (b is None):
            return float("inf")
        if a is not None:
            worst = max(worst, float(np.abs(a - b).max()))
    return worst


def window1_err(mod, scale=0.53):
    q, k, v, do, sink = inputs(2, 9, 4, 2, 6, 5, True, seed=7)
    G = 2
    dq, dk, dv, ds = mod.prefill_backward(q, k, v, do, 1, sink, scale)
    eq, ek, ev, es = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros(4)
    for b in range(2):
        for i in range(9):
            for h in range(4):
                g = h // G
                sig = 1.0 / (1.0 + np.exp(-(scale * q[b, i, h] @ k[b, i, g] - sink[h])))
                a = do[b, i, h] @ v[b, i, g]  # dLoss/d(weight) of the one real key
                w = sig * (1 - sig) * a       # dLoss/d(score)
                eq[b, i, h] = scale * w * k[b, i, g]
                ek[b, i, g] += scale * w * q[b, i, h]
                ev[b, i, g] += sig * do[b, i, h]
                es[h] -= w
    return max(float(np.abs(x - y).max()) for x, y in ((dq, eq), (dk, ek), (dv, ev), (ds, es)))


def identity_errs(mod, window, with_sink, scale=0.2):
    q, k, v, do, sink = inputs(2, 150, 8, 4, 16, 8, with_sink, seed=300 + window)
    dq, dk, dv, _ = mod.prefill_backward(q, k, v, do, window, sink, scale, block=64)
    o, _ = oracle.prefill(q, k, v, window, sink, scale)
    bil = abs((q * dq).sum() - (k * dk).sum()) / (1 + abs((q * dq).sum()))
    lin = abs((v * dv).sum() - (do * o).sum()) / (1 + abs((do * o).sum()))
    shift = 0.0 if with_sink else float(np.abs(dk.sum(axis=1)).max())
    return bil, lin, shift


def run_pins(mod):
    failed = []
    for window in (1, 3, 100):
        for with_sink in (True, False):
            if fd_err(mod, window, with_sink) > 1e-7:
                failed.append(f"finite differences W={window} sink={with_sink}")
    for window in (16, 1000):
        for with_sink in (True, False):
            if autograd_err(mod, window, with_sink) > 1e-11:
                failed.append(f"autograd W={window} sink={with_sink}")
    if window1_err(mod) > 1e-12:
        failed.append("window-1 closed form")
    for window in (20, 1000):
        for with_sink in (True, False):
            bil, lin, shift = identity_errs(mod, window, with_sink)
            if bil > 1e-11 or lin > 1e-11 or shift > 1e-10:
                failed.append(f"identities W={window} sink={with_sink}")
    return failed


def test_pins_pass_on_the_oracle():
    assert run_pins(ob) == []


def test_sink_gradient_matches_its_definition():
    # d loss / d s_h = -sum_i p_sink_i D_i, with D_i = dO_i . o_i and p_sink_i = exp(s_h - lse_i)
    q, k, v, do, sink = inputs(2, 40, 4, 2, 8, 6, True, seed=11)
    _, _, _, ds = oracle.prefill_backward(q, k, v, do, 9, sink, 0.3)
    o, lse = oracle.prefill(q, k, v, 9, sink, 0.3)
    D = np.einsum("bihd,bihd->bhi", do, o)
    expect = -(np.exp(sink[None, :, None] - lse) * D).sum(axis=(0, 2))
    np.testing.assert_allclose(ds, expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [5, 64, 10**9])
def test_row_and_key_samplers_match_the_whole_tensor(window):
    q, k, v, do, sink = inputs(2, 90, 8, 2, 10, 6, True, seed=window % 97)
    dq, dk, dv, _ = oracle.prefill_backward(q, k, v, do, window, sink, 0.25, block=40)
    rows = [(0, 0), (1, 5), (0, 63), (1, 89)]
    got = oracle.backward_rows(q, k, v, do, window, sink, 0.25, rows)
    for n, (b, i) in enumerate(rows):
        np.testing.assert_allclose(got[n], dq[b, i], rtol=1e-12, atol=1e-12)
    keys = [(0, 0), (1, 1), (0, 44), (1, 89)]
    gk, gv = oracle.backward_keys(q, k, v, do, window, sink, 0.25, keys)
    for n, (b, j) in enumerate(keys):
        np.testing.assert_allclose(gk[n], dk[b, j], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gv[n], dv[b, j], rtol=1e-12, atol=1e-12)


def test_no_sink_gives_no_sink_gradient():
    q, k, v, do, _ = inputs(1, 10, 2, 1, 4, 3, False)
    assert oracle.prefill_backward(q, k, v, do, 4, None, 0.5)[3] is None


# ------------------------------------------------------------------------------ planted mistakes

class Mutant:
    """The gradient oracle with one planted mistake."""

    def __init__(self, fn):
        self.prefill_backward = fn


def _no_sink_weights(*a, **kw):
    q, k, v, do, window, sink, scale = a[:7]
    return ob.prefill_backward(q, k, v, do, window, None, scale, **kw)[:3] + (
        ob.prefill_backward(q, k, v, do, window, sink, scale, **kw)[3],)


def _flipped_sink_sign(*a, **kw):
    dq, dk, dv, ds = ob.prefill_backward(*a, **kw)
    return dq, dk, dv, (None if ds is None else -ds)


def _dk_without_scale(*a, **kw):
    dq, dk, dv, ds = ob.prefill_backward(*a, **kw)
    return dq, dk / a[6], dv, ds


def _wrong_gqa(*a, **kw):
    q, k = a[0], a[1]
    Hq, Hkv = q.shape[2], k.shape[2]
    return ob.prefill_backward(*a, kv_head_of_q=np.arange(Hq) % Hkv, **kw)


def _raw_dp_sum(q_rows, q_pos, keys, k_pos, vals, do_rows, sink_h, scale, window, real=ob._row_terms):
    p, p_sink, D, ds = real(q_rows, q_pos, keys, k_pos, vals, do_rows, sink_h, scale, window)
    dp = do_rows @ vals.T
    vis = p > 0
    D2 = np.where(vis, dp, 0.0).sum(axis=1) / np.maximum(vis.sum(axis=1), 1)  # mean instead of p-weighted
    return p, p_sink, D2, p * (dp - D2[:, None])


@pytest.mark.parametrize("name", ["no sink weights", "sink sign", "dk scale", "gqa map", "raw dp"])
def test_planted_mistakes_are_caught(name, monkeypatch):
    if name == "raw dp":
        monkeypatch.setattr(ob, "_row_terms", _raw_dp_sum)
        mod = ob
    else:
        mod = Mutant({"no sink weights": _no_sink_weights, "sink sign": _flipped_sink_sign,
                      "dk scale": _dk_without_scale, "gqa map": _wrong_gqa}[name])
    assert run_pins(mod) != [], name
