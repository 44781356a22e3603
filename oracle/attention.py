"""Float64 CPU oracle for sink-seeded sliding-window and global attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check and the bench's
CPU-baseline leg may import, call or run anything in this package. It shares no code with the HIP
library and imports nothing from it; it receives plain numpy arrays.

What is computed, and where the pages say so
--------------------------------------------
* MiMo-V2-Flash Technical Report review (xllm-io paper review), §3.1: sliding-window layers use a
  window of W = 128 tokens; GQA with 64 query heads over 8 KV heads (SWA) or 4 KV heads (global);
  head dims 192 for Q/K and 128 for V.
* Same page, §3.2, and the MiMo series notes (plmsmile), MiMo-V2-Flash > Learnable Attention Sink >
  mechanism: every attention head adds a learnable sink term to its softmax denominator, so the
  weights of the real tokens may sum to less than one; the sink carries no text and only sets how
  strongly the head outputs its real values.
* MiMo series notes, MiMo-V2-Flash > local window: a sliding-window layer reads only the 128
  neighbouring tokens. jienda explainer §2.1: each token attends to the 128 tokens in front of it.
* MiMo series notes, MiMo-V2-Flash > lightweight MTP > inference: draft tokens are verified by the
  main model in parallel, i.e. a decode step carries 1 + drafts query tokens per sequence.

Readings taken where the pages are silent (all listed again in the design notes):
* The sink enters the denominator as exp(s_h) for query head h (a real-valued logit, never scaled
  by the softmax scale); it contributes a zero value vector.
* Key j is visible to query i iff 0 <= i - j < W (W keys including the query's own);
  W >= L is plain causal (global) attention.
* The softmax scale multiplies q.k only. The GQA map is contiguous (g = h // (Hq/Hkv)) unless an
  explicit map is given.
* Decode: the cache holds committed positions only; position p of sequence b lives in slot
  (p + off_b) mod C; the T new tokens sit at positions P_b .. P_b+T-1 and draft t sees new tokens
  0..t.
* LSE is the natural log of the full denominator, sink included.

Per output row i of head h (plain definition, evaluated with a max shift for range only):
    s_ij = scale * <q_i, k_j>                  for visible j
    m_i  = max(s_h, max_j s_ij)
    Z_i  = exp(s_h - m_i) + sum_j exp(s_ij - m_i)
    o_i  = sum_j exp(s_ij - m_i) / Z_i * v_j
    lse_i = m_i + log Z_i

Every function here is pinned by tests that do not reuse this code (brute force in mpmath, a
library attention routine with the sink posed as an extra key, closed forms and invariants).
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def default_kv_map(Hq: int, Hkv: int) -> np.ndarray:
    """Contiguous GQA grouping: query head h reads KV head h // (Hq / Hkv)."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return np.arange(Hq) // (Hq // Hkv)


def visible(q_pos: np.ndarray, k_pos: np.ndarray, window: int) -> np.ndarray:
    """[n, m] boolean: key position k_pos[j] is visible to query position q_pos[i]."""
    d = q_pos[:, None] - k_pos[None, :]
    return (d >= 0) & (d < window)


def sink_attention(q_rows, q_pos, keys, k_pos, vals, sink_h, scale, window):
    """The definition for one head: q_rows [n, dqk], keys [m, dqk], vals [m, dv].

    Returns (o [n, dv], lse [n], lse_real [n]); lse includes the sink, lse_real only the keys.
    ``sink_h`` is a float (may be -inf for "no sink").
    """
    q_rows, keys, vals = _f64(q_rows), _f64(keys), _f64(vals)
    s = scale * (q_rows @ keys.T)
    vis = visible(np.asarray(q_pos), np.asarray(k_pos), window)
    if not vis.any(axis=1).all():
        raise ValueError("a query row sees no key")
    s = np.where(vis, s, NEG_INF)
    row_max = s.max(axis=1)
    m = np.maximum(row_max, sink_h)
    e = np.exp(s - m[:, None])
    z = np.exp(sink_h - m) + e.sum(axis=1)
    o = (e / z[:, None]) @ vals
    lse = m + np.log(z)
    lse_real = row_max + np.log(np.exp(s - row_max[:, None]).sum(axis=1))
    return o, lse, lse_real


def _sink_value(sink, h):
    return NEG_INF if sink is None else float(sink[h])


def prefill_rows(q, k, v, window, sink, scale, rows, kv_head_of_q=None, return_real=False):
    """Outputs for selected query positions.

    q [B, L, Hq, dqk], k [B, L, Hkv, dqk], v [B, L, Hkv, dv] (any float dtype, read exactly);
    rows: sequence of (b, i). Returns o [n, Hq, dv] and lse [n, Hq] in float64.
    """
    B, L, Hq, _ = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    kvm = default_kv_map(Hq, Hkv) if kv_head_of_q is None else np.asarray(kv_head_of_q)
    rows = [(int(b), int(i)) for b, i in rows]
    o = np.empty((len(rows), Hq, dv))
    lse = np.empty((len(rows), Hq))
    lse_r = np.empty((len(rows), Hq))
    for n, (b, i) in enumerate(rows):
        lo = max(0, i - window + 1)
        k_pos = np.arange(lo, i + 1)
        for h in range(Hq):
            g = kvm[h]
            oo, ll, lr = sink_attention(q[b, i:i + 1, h], np.array([i]), k[b, lo:i + 1, g], k_pos,
                                        v[b, lo:i + 1, g], _sink_value(sink, h), scale, window)
            o[n, h], lse[n, h], lse_r[n, h] = oo[0], ll[0], lr[0]
    if return_real:
        return o, lse, lse_r
    return o, lse


def prefill(q, k, v, window, sink, scale, kv_head_of_q=None, block=256, return_real=False):
    """Whole-tensor prefill: o [B, L, Hq, dv], lse [B, Hq, L] (float64).

    Rows are taken in blocks of ``block`` positions; each block sees keys
    [max(0, i0 - W + 1), i1) and the visibility predicate does the rest.
    """
    B, L, Hq, _ = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    kvm = default_kv_map(Hq, Hkv) if kv_head_of_q is None else np.asarray(kv_head_of_q)
    o = np.empty((B, L, Hq, dv))
    lse = np.empty((B, Hq, L))
    lse_r = np.empty((B, Hq, L))
    for b in range(B):
        for i0 in range(0, L, block):
            i1 = min(L, i0 + block)
            lo = max(0, i0 - window + 1)
            q_pos, k_pos = np.arange(i0, i1), np.arange(lo, i1)
            for h in range(Hq):
                g = kvm[h]
                oo, ll, lr = sink_attention(q[b, i0:i1, h], q_pos, k[b, lo:i1, g], k_pos,
                                            v[b, lo:i1, g], _sink_value(sink, h), scale, window)
                o[b, i0:i1, h], lse[b, h, i0:i1], lse_r[b, h, i0:i1] = oo, ll, lr
    if return_real:
        return o, lse, lse_r
    return o, lse


def decode_keys(k_new, v_new, k_cache, v_cache, b, P, off, window, T):
    """Logical key/value sequence that the T new queries of sequence b can see.

    Committed positions [max(0, P - W + 1), P) are read from ring slot (p + off) mod C; the new
    tokens follow at positions P .. P+T-1. Returns (k_pos, keys [m, Hkv, dqk], vals [m, Hkv, dv]).
    """
    C = k_cache.shape[1]
    lo = max(0, P - window + 1)
    if P - lo > C:
        raise ValueError("cache too small for the window: committed keys were overwritten")
    pos = np.arange(lo, P)
    slots = (pos + off) % C
    keys = np.concatenate([k_cache[b, slots], k_new[b, :T]], axis=0)
    vals = np.concatenate([v_cache[b, slots], v_new[b, :T]], axis=0)
    k_pos = np.concatenate([pos, np.arange(P, P + T)])
    return k_pos, keys, vals


def decode(q, k_new, v_new, k_cache, v_cache, cache_len, cache_offset, window, sink, scale,
           kv_head_of_q=None, seqs=None, heads=None, return_real=False):
    """Decode with T = q.shape[1] new tokens per sequence.

    Returns o [B, T, Hq, dv] and lse [B, T, Hq] in float64 (rows of sequences/heads not selected by
    ``seqs``/``heads`` are left as NaN).
    """
    B, T, Hq, _ = q.shape
    Hkv, dv = k_new.shape[2], v_new.shape[3]
    kvm = default_kv_map(Hq, Hkv) if kv_head_of_q is None else np.asarray(kv_head_of_q)
    o = np.full((B, T, Hq, dv), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    lse_r = np.full((B, T, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        P = int(cache_len[b])
        off = 0 if cache_offset is None else int(cache_offset[b])
        k_pos, keys, vals = decode_keys(k_new, v_new, k_cache, v_cache, b, P, off, window, T)
        q_pos = np.arange(P, P + T)
        for h in (range(Hq) if heads is None else heads):
            g = kvm[h]
            oo, ll, lr = sink_attention(q[b, :, h], q_pos, keys[:, g], k_pos, vals[:, g],
                                        _sink_value(sink, h), scale, window)
            o[b, :, h], lse[b, :, h], lse_r[b, :, h] = oo, ll, lr
    if return_real:
        return o, lse, lse_r
    return o, lse


def split_partials(q_rows, q_pos, keys, k_pos, vals, scale, window, num_splits):
    """Split-KV partials over contiguous key chunks, without the sink.

    For chunk c: m_c = max visible score (-inf if none), l_c = sum exp(s - m_c),
    acc_c = sum exp(s - m_c) v. Returns lists (m, l, acc).
    """
    q_rows, keys, vals = _f64(q_rows), _f64(keys), _f64(vals)
    n, m_keys = q_rows.shape[0], keys.shape[0]
    bounds = np.linspace(0, m_keys, num_splits + 1).round().astype(int)
    ms, ls, accs = [], [], []
    for c in range(num_splits):
        a, z = bounds[c], bounds[c + 1]
        if z <= a:
            ms.append(np.full(n, NEG_INF)), ls.append(np.zeros(n)), accs.append(np.zeros((n, vals.shape[1])))
            continue
        s = scale * (q_rows @ keys[a:z].T)
        s = np.where(visible(np.asarray(q_pos), np.asarray(k_pos[a:z]), window), s, NEG_INF)
        mc = s.max(axis=1)
        safe = np.where(np.isfinite(mc), mc, 0.0)
        e = np.exp(s - safe[:, None])
        ms.append(mc), ls.append(e.sum(axis=1)), accs.append(e @ vals[a:z])
    return ms, ls, accs


def combine(ms, ls, accs, sink_h):
    """Fold split partials and the sink (counted once): returns (o, lse)."""
    M = np.maximum.reduce([np.full_like(ms[0], sink_h)] + list(ms))
    Z = np.exp(sink_h - M)
    acc = np.zeros_like(accs[0])
    for mc, lc, ac in zip(ms, ls, accs):
        w = np.where(np.isfinite(mc), np.exp(np.where(np.isfinite(mc), mc, 0.0) - M), 0.0)
        Z = Z + lc * w
        acc = acc + ac * w[:, None]
    return acc / Z[:, None], M + np.log(Z)
