"""Float64 CPU oracle for the gradients of sink-seeded attention (the training backward pass).

TEST INFRASTRUCTURE, NOT PRODUCT CODE (same rules as ``oracle.attention``): only the test suite,
the smoke check and the bench's CPU-baseline leg may import it; it shares no code with the HIP
library.

What the pages fix
------------------
* MiMo-V2-Flash Technical Report review (xllm-io), §3.2, and MiMo series notes (plmsmile),
  MiMo-V2-Flash > Learnable Attention Sink: the sink value s_h of each head is a learned
  parameter, so training needs its gradient next to those of Q, K and V.
* The forward operation is the one of ``oracle.attention`` (window, GQA, sink in the denominator
  with no value vector, scale on q.k only).

Gradients of a scalar loss with upstream gradient dO = dLoss/dO, written out from the chain rule
of the forward definition (row i of query head h, visible keys j, KV head g of h):
    p_ij   = exp(s_ij - lse_i)                    real-key weights
    p^s_i  = exp(s_h - lse_i)                     the sink's weight (its value vector is zero)
    dp_ij  = <dO_i, v_j>
    D_i    = sum_j p_ij dp_ij  (= <dO_i, o_i>)     the sink adds p^s_i * 0
    ds_ij  = p_ij (dp_ij - D_i)                   gradient of the score s_ij
    dq_i   = scale * sum_j ds_ij k_j
    dk_j   = scale * sum_{h in g} sum_i ds_ij q_i      (summed over the query heads of g)
    dv_j   = sum_{h in g} sum_i p_ij dO_i
    ds_h   = -sum_{b, i} p^s_i D_i               gradient of the sink logit

Readings taken where the pages are silent (listed again in the design notes):
* The loss is any scalar; the oracle takes its gradient dO with respect to the attention output.
* The gradient of the sink sums over every sequence of the batch and every query row.

Pinned by tests that do not reuse this code: central finite differences of the forward oracle,
a closed form at window 1 (the softmax over one key and the sink is a logistic function),
identities that hold at any size, and planted mistakes that those pins catch.
"""

from __future__ import annotations

import numpy as np

from .attention import NEG_INF, default_kv_map, visible


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _row_terms(q_rows, q_pos, keys, k_pos, vals, do_rows, sink_h, scale, window):
    """p [n, m], p_sink [n], ds [n, m] for one head over a block of rows and its keys."""
    s = scale * (q_rows @ keys.T)
    vis = visible(np.asarray(q_pos), np.asarray(k_pos), window)
    if not vis.any(axis=1).all():
        raise ValueError("a query row sees no key")
    s = np.where(vis, s, NEG_INF)
    m = np.maximum(s.max(axis=1), sink_h)
    e = np.exp(s - m[:, None])
    es = np.exp(sink_h - m)
    z = es + e.sum(axis=1)
    p = e / z[:, None]
    p_sink = es / z
    dp = do_rows @ vals.T
    D = (p * dp).sum(axis=1)
    ds = p * (dp - D[:, None])
    return p, p_sink, D, ds


def _sink_value(sink, h):
    return NEG_INF if sink is None else float(sink[h])


def prefill_backward(q, k, v, do, window, sink, scale, kv_head_of_q=None, block=256):
    """Gradients of a prefill: (dq [B, L, Hq, dqk], dk [B, L, Hkv, dqk], dv [B, L, Hkv, dv],
    dsink [Hq] or None when there is no sink), all float64.

    q, k, v as for ``oracle.prefill``; do [B, L, Hq, dv] is the upstream gradient of the output.
    Rows are taken in blocks of ``block`` positions, each with the keys its window reaches.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, L, Hq, _ = q.shape
    Hkv = k.shape[2]
    kvm = default_kv_map(Hq, Hkv) if kv_head_of_q is None else np.asarray(kv_head_of_q)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsink = np.zeros(Hq)
    for b in range(B):
        for i0 in range(0, L, block):
            i1 = min(L, i0 + block)
            lo = max(0, i0 - window + 1)
            q_pos, k_pos = np.arange(i0, i1), np.arange(lo, i1)
            for h in range(Hq):
                g = kvm[h]
                p, p_sink, D, ds = _row_terms(q[b, i0:i1, h], q_pos, k[b, lo:i1, g], k_pos,
                                              v[b, lo:i1, g], do[b, i0:i1, h], _sink_value(sink, h),
                                              scale, window)
                dq[b, i0:i1, h] = scale * (ds @ k[b, lo:i1, g])
                dk[b, lo:i1, g] += scale * (ds.T @ q[b, i0:i1, h])
                dv[b, lo:i1, g] += p.T @ do[b, i0:i1, h]
                dsink[h] -= (p_sink * D).sum()
    return dq, dk, dv, (None if sink is None else dsink)


def backward_rows(q, k, v, do, window, sink, scale, rows, kv_head_of_q=None):
    """dq of selected query rows: rows = [(b, i)]; returns [n, Hq, dqk] (float64).

    Inputs may be any float arrays; only the slices a row needs are read (and widened).
    """
    Hq = q.shape[2]
    kvm = default_kv_map(Hq, k.shape[2]) if kv_head_of_q is None else np.asarray(kv_head_of_q)
    out = np.empty((len(rows), Hq, q.shape[3]))
    for n, (b, i) in enumerate(rows):
        lo = max(0, i - window + 1)
        qs, ks, vs, ds_ = (_f64(x[b, a:z]) for x, a, z in
                           ((q, i, i + 1), (k, lo, i + 1), (v, lo, i + 1), (do, i, i + 1)))
        for h in range(Hq):
            g = kvm[h]
            _, _, _, ds = _row_terms(qs[:, h], [i], ks[:, g], np.arange(lo, i + 1), vs[:, g],
                                     ds_[:, h], _sink_value(sink, h), scale, window)
            out[n, h] = scale * (ds @ ks[:, g])[0]
    return out


def backward_keys(q, k, v, do, window, sink, scale, keys, kv_head_of_q=None):
    """dk and dv of selected key positions: keys = [(b, j)]; returns ([n, Hkv, dqk], [n, Hkv, dv]).

    Key j receives from query rows i in [j, min(L, j + W)); each such row's weights are computed
    over that row's whole window. Only the slices those rows need are read (and widened).
    """
    L, Hq, Hkv = q.shape[1], q.shape[2], k.shape[2]
    kvm = default_kv_map(Hq, Hkv) if kv_head_of_q is None else np.asarray(kv_head_of_q)
    dk = np.zeros((len(keys), Hkv, k.shape[3]))
    dv = np.zeros((len(keys), Hkv, v.shape[3]))
    for n, (b, j) in enumerate(keys):
        i0, i1 = j, min(L, j + window)
        lo = max(0, i0 - window + 1)
        q_pos, k_pos = np.arange(i0, i1), np.arange(lo, i1)
        qs, ks, vs, ds_ = (_f64(x[b, a:z]) for x, a, z in
                           ((q, i0, i1), (k, lo, i1), (v, lo, i1), (do, i0, i1)))
        col = j - lo
        for h in range(Hq):
            g = kvm[h]
            p, _, _, ds = _row_terms(qs[:, h], q_pos, ks[:, g], k_pos, vs[:, g], ds_[:, h],
                                     _sink_value(sink, h), scale, window)
            dk[n, g] += scale * (ds[:, col] @ qs[:, h])
            dv[n, g] += p[:, col] @ ds_[:, h]
    return dk, dv
