"""Pins for the float64 oracle: each check compares it with something that is not the oracle.

* mpmath brute force at 50 digits of the textbook formula (no max shift, keys enumerated as a range);
* torch's scaled_dot_product_attention (CPU, float64) with the sink posed as one extra key whose
  score is the unscaled sink logit and whose value is zero (MiMo series notes, MiMo-V2-Flash >
  Learnable Attention Sink > mechanism: the sink joins the denominator and carries no content);
* the library's own causal mask and GQA grouping when there is no sink;
* closed forms (W = 1, L = 1, a dominant sink) and invariants (row mass, output range, window
  slices, GQA = MHA with repeated KV, decode rows = prefill tail rows, split invariance).

The mutation tests at the end plant plausible mistakes in the oracle and require that a pin fails.
"""

import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa

RNG = np.random.default_rng(12345)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# ---------------------------------------------------------------- pin helpers (return max error)

def brute_force_err(mod, B, L, Hq, Hkv, dqk, dv, window, sink, scale, peaky=1.0):
    """mpmath 50-digit evaluation of o = sum_j e^{s_ij} v_j / (e^{s_h} + sum_j e^{s_ij})."""
    q, k, v = rand(B, L, Hq, dqk, scale=peaky), rand(B, L, Hkv, dqk), rand(B, L, Hkv, dv)
    o, lse = mod.prefill(q, k, v, window, sink, scale)
    G = Hq // Hkv
    worst = 0.0
    with mpmath.workdps(50):
        for b in range(B):
            for h in range(Hq):
                g = h // G
                for i in range(L):
                    num = [mpmath.mpf(0)] * dv
                    den = mpmath.mpf(0) if sink is None else mpmath.exp(mpmath.mpf(float(sink[h])))
                    for j in range(max(0, i - window + 1), i + 1):
                        s = mpmath.mpf(scale) * mpmath.fsum(
                            mpmath.mpf(float(q[b, i, h, d])) * mpmath.mpf(float(k[b, j, g, d]))
                            for d in range(dqk))
                        e = mpmath.exp(s)
                        den += e
                        for d in range(dv):
                            num[d] += e * mpmath.mpf(float(v[b, j, g, d]))
                    for d in range(dv):
                        worst = max(worst, abs(float(num[d] / den) - o[b, i, h, d]))
                    worst = max(worst, abs(float(mpmath.log(den)) - lse[b, h, i]))
    return worst


def sdpa_extra_key_err(mod, B, L, Hq, Hkv, dqk, dv, window, sink, scale):
    q, k, v = rand(B, L, Hq, dqk), rand(B, L, Hkv, dqk), rand(B, L, Hkv, dv)
    o, _ = mod.prefill(q, k, v, window, sink, scale)
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)  # [B, Hq, L, d]
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    # append the sink as key L: zero key (score 0) plus an additive mask equal to s_h, zero value
    tk = torch.cat([tk, torch.zeros(B, Hq, 1, dqk, dtype=torch.float64)], dim=2)
    tv = torch.cat([tv, torch.zeros(B, Hq, 1, dv, dtype=torch.float64)], dim=2)
    ones = torch.ones(L, L, dtype=torch.bool)
    keep = torch.tril(ones) & ~torch.tril(ones, diagonal=-window)  # j <= i and j > i - W
    mask = torch.full((Hq, L, L + 1), -math.inf, dtype=torch.float64)
    mask[:, :, :L][keep.expand(Hq, L, L)] = 0.0
    mask[:, :, L] = torch.from_numpy(np.asarray(sink, dtype=np.float64))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    return float(np.abs(ref.permute(0, 2, 1, 3).numpy() - o).max())


def causal_sdpa_err(mod, B, L, Hq, Hkv, dqk, dv, sink, scale):
    q, k, v = rand(B, L, Hq, dqk), rand(B, L, Hkv, dqk), rand(B, L, Hkv, dv)
    o, _ = mod.prefill(q, k, v, L, sink, scale)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True,
                                                           scale=scale, enable_gqa=True)
    return float(np.abs(ref.permute(0, 2, 1, 3).numpy() - o).max())


def window1_err(mod, L, Hq, Hkv, dqk, dv, sink, scale):
    q, k, v = rand(1, L, Hq, dqk), rand(1, L, Hkv, dqk), rand(1, L, Hkv, dv)
    o, lse = mod.prefill(q, k, v, 1, sink, scale)
    G = Hq // Hkv
    worst = 0.0
    for h in range(Hq):
        for i in range(L):
            s = scale * float(q[0, i, h] @ k[0, i, h // G])
            w = 1.0 / (1.0 + math.exp(float(sink[h]) - s))  # sigma(s_ii - s_h)
            worst = max(worst, float(np.abs(o[0, i, h] - w * v[0, i, h // G]).max()))
            worst = max(worst, abs(lse[0, h, i] - np.logaddexp(float(sink[h]), s)))
    return worst


def decode_tail_err(mod, P, T, off, C, window, Hq=4, Hkv=2, dqk=8, dv=5, scale=0.37):
    """Decode rows must equal the last T prefill rows of the unrolled sequence."""
    n = P + T
    kf, vf, q = rand(1, n, Hkv, dqk), rand(1, n, Hkv, dv), rand(1, n, Hq, dqk)
    sink = rand(Hq)
    k_cache, v_cache = rand(1, C, Hkv, dqk) * 50, rand(1, C, Hkv, dv) * 50  # stale slots: garbage
    for pos in range(max(0, P - C), P):  # forward mapping: write committed positions into the ring
        k_cache[0, (pos + off) % C] = kf[0, pos]
        v_cache[0, (pos + off) % C] = vf[0, pos]
    o_dec, lse_dec = mod.decode(q[:, P:], kf[:, P:], vf[:, P:], k_cache, v_cache,
                                np.array([P]), np.array([off]), window, sink, scale)
    o_pre, lse_pre = mod.prefill(q, kf, vf, window, sink, scale)
    e1 = np.abs(o_dec[0] - o_pre[0, P:]).max()
    e2 = np.abs(lse_dec[0] - lse_pre[0, :, P:].T).max()
    return float(max(e1, e2))


def row_mass_err(mod, L, Hq, Hkv, dqk, window, sink, scale):
    q, k = rand(1, L, Hq, dqk), rand(1, L, Hkv, dqk)
    ones = np.ones((1, L, Hkv, 1))
    mass, lse, lse_real = mod.prefill(q, k, ones, window, sink, scale, return_real=True)
    mass = mass[0, :, :, 0].T  # [Hq, L]
    s_h = np.full((Hq, 1), -np.inf) if sink is None else np.asarray(sink)[:, None]
    e1 = np.abs(mass - 1.0 / (1.0 + np.exp(s_h - lse_real[0]))).max()
    e2 = np.abs(mass - (1.0 - np.exp(s_h - lse[0]))).max()
    return float(max(e1, e2)), mass


# ---------------------------------------------------------------- the pins

@pytest.mark.parametrize("L,Hq,Hkv,dqk,dv", [(5, 2, 1, 3, 2), (8, 4, 2, 4, 3), (1, 2, 2, 2, 2)])
def test_mpmath_bruteforce_every_window(L, Hq, Hkv, dqk, dv):
    for window in range(1, L + 2):
        for sink in (None, rand(Hq)):
            assert brute_force_err(oracle, 1, L, Hq, Hkv, dqk, dv, window, sink, 0.7) < 1e-13


def test_mpmath_bruteforce_peaky_and_extreme_sinks():
    sink = np.array([30.0, -30.0, 0.0, 5.0])
    assert brute_force_err(oracle, 2, 6, 4, 2, 4, 3, 3, sink, 0.5, peaky=8.0) < 1e-12


@pytest.mark.parametrize("window", [1, 2, 3, 7, 16, 40])
def test_sdpa_with_sink_as_extra_key(window):
    assert sdpa_extra_key_err(oracle, 2, 23, 8, 2, 16, 12, window, rand(8), 0.25) < 1e-12


@pytest.mark.parametrize("sink", [None, np.full(6, -np.inf)])
def test_no_sink_is_library_causal_attention(sink):
    assert causal_sdpa_err(oracle, 2, 19, 6, 3, 12, 7, sink, 0.3) < 1e-12


def test_dominant_sink_zeroes_the_output():
    q, k, v = rand(1, 9, 2, 4), rand(1, 9, 1, 4), rand(1, 9, 1, 3)
    o, lse = oracle.prefill(q, k, v, 4, np.array([1e4, 1e4]), 1.0)
    assert np.all(o == 0.0)
    assert np.allclose(lse, 1e4, rtol=0, atol=1e-9)


def test_window_one_closed_form():
    assert window1_err(oracle, 11, 4, 2, 6, 5, rand(4), 0.4) < 1e-13


def test_single_token_closed_form():
    q, k, v = rand(1, 1, 3, 5), rand(1, 1, 3, 5), rand(1, 1, 3, 4)
    sink = rand(3)
    for window in (1, 128):
        o, lse = oracle.prefill(q, k, v, window, sink, 0.9)
        for h in range(3):
            s = 0.9 * float(q[0, 0, h] @ k[0, 0, h])
            np.testing.assert_allclose(o[0, 0, h], v[0, 0, h] / (1 + math.exp(sink[h] - s)),
                                       rtol=1e-14, atol=1e-15)


def test_window_at_least_length_is_global():
    q, k, v = rand(2, 13, 4, 5), rand(2, 13, 2, 5), rand(2, 13, 2, 3)
    sink = rand(4)
    ref, ref_lse = oracle.prefill(q, k, v, 13, sink, 0.5)
    for window in (14, 128, 10**9):
        o, lse = oracle.prefill(q, k, v, window, sink, 0.5)
        assert np.array_equal(o, ref) and np.array_equal(lse, ref_lse)


def test_swa_row_is_global_attention_on_its_window():
    L, W = 30, 7
    q, k, v = rand(1, L, 2, 4), rand(1, L, 1, 4), rand(1, L, 1, 3)
    sink = rand(2)
    o, _ = oracle.prefill(q, k, v, W, sink, 0.6)
    for i in range(L):
        lo = max(0, i - W + 1)
        og, _ = oracle.prefill(q[:, lo:i + 1], k[:, lo:i + 1], v[:, lo:i + 1], 10**6, sink, 0.6)
        np.testing.assert_allclose(o[0, i], og[0, -1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("window", [1, 5, 64])
def test_row_mass_below_one_and_matches_sigmoid(window):
    sink = rand(4)
    err, mass = row_mass_err(oracle, 40, 4, 2, 8, window, sink, 0.35)
    assert err < 1e-13
    assert np.all(mass < 1.0) and np.all(mass > 0.0)
    err, mass = row_mass_err(oracle, 40, 4, 2, 8, window, None, 0.35)
    assert err < 1e-13 and np.allclose(mass, 1.0, atol=1e-14)


def test_output_inside_mass_scaled_value_hull():
    L, W = 25, 6
    q, k, v = rand(1, L, 2, 4), rand(1, L, 1, 4), rand(1, L, 1, 3)
    sink = rand(2)
    o, _ = oracle.prefill(q, k, v, W, sink, 0.8)
    mass, _ = oracle.prefill(q, k, np.ones((1, L, 1, 1)), W, sink, 0.8)
    for i in range(L):
        win = v[0, max(0, i - W + 1):i + 1, 0]
        for h in range(2):
            m = mass[0, i, h, 0]
            assert np.all(o[0, i, h] <= m * win.max(0) + 1e-14)
            assert np.all(o[0, i, h] >= m * win.min(0) - 1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = rand(2, 17, 8, 6), rand(2, 17, 2, 6), rand(2, 17, 2, 4)
    sink = rand(8)
    o, lse = oracle.prefill(q, k, v, 5, sink, 0.4)
    o2, lse2 = oracle.prefill(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 5, sink, 0.4)
    assert np.abs(o - o2).max() < 1e-15 and np.abs(lse - lse2).max() < 1e-15


def test_explicit_kv_map_is_a_head_permutation():
    q, k, v = rand(1, 12, 6, 4), rand(1, 12, 3, 4), rand(1, 12, 3, 2)
    sink = rand(6)
    perm = np.array([3, 0, 5, 1, 4, 2])
    base, base_lse = oracle.prefill(q, k, v, 4, sink, 0.5)  # contiguous map: h // 2
    kvm = perm // 2  # head j of the permuted problem is head perm[j] of the base one
    o, lse = oracle.prefill(q[:, :, perm], k, v, 4, sink[perm], 0.5, kv_head_of_q=kvm)
    assert np.abs(o - base[:, :, perm]).max() < 1e-15
    assert np.abs(lse - base_lse[:, perm]).max() < 1e-15


@pytest.mark.parametrize("P", [0, 1, 5, 126, 127, 128, 1000])
@pytest.mark.parametrize("T", [1, 2, 4])
def test_decode_is_prefill_tail_on_a_ring(P, T):
    for off in (0, 1, 63, 127) if P > 5 else range(128):
        assert decode_tail_err(oracle, P, T, off, 128, 128) < 1e-12


def test_decode_small_ring_and_window():
    # C = W - 1 is the smallest cache that still holds every visible committed key
    for P in range(0, 20):
        for off in range(6):
            assert decode_tail_err(oracle, P, 3, off, 6, 7) < 1e-12


def test_decode_global_linear_cache():
    for P in (0, 3, 200):
        assert decode_tail_err(oracle, P, 4, 0, 256, 10**9) < 1e-12


def test_decode_rejects_overwritten_window():
    with pytest.raises(ValueError):
        decode_tail_err(oracle, 50, 1, 0, 8, 20)


@pytest.mark.parametrize("num_splits", [1, 2, 7, 40, 300])
def test_split_combine_equals_single_pass(num_splits):
    n, m = 4, 211
    q, keys, vals = rand(n, 6), rand(m, 6), rand(m, 5)
    q_pos = np.arange(m - n, m)
    k_pos = np.arange(m)
    for sink_h in (-np.inf, 0.3, 40.0):
        for window in (m, 50):
            o, lse, _ = oracle.sink_attention(q, q_pos, keys, k_pos, vals, sink_h, 0.45, window)
            ms, ls, accs = oracle.split_partials(q, q_pos, keys, k_pos, vals, 0.45, window, num_splits)
            oc, lsec = oracle.combine(ms, ls, accs, sink_h)
            assert np.abs(o - oc).max() < 1e-12 and np.abs(lse - lsec).max() < 1e-12


def test_shape_facts_match_the_pages():
    import json
    import os
    from sliding_window_sink_seeded_amd import workloads

    facts = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.json")))
    swa, ga = workloads.WORKLOADS["swa_prefill_bf16"], workloads.WORKLOADS["ga_prefill_bf16"]
    assert swa.window == facts["window"]["value"]
    assert (swa.Hq, swa.Hkv) == (facts["swa_q_heads"]["value"], facts["swa_kv_heads"]["value"])
    assert (ga.Hq, ga.Hkv) == (facts["ga_q_heads"]["value"], facts["ga_kv_heads"]["value"])
    for w in workloads.WORKLOADS.values():
        assert (w.dqk, w.dv) == (facts["d_qk"]["value"], facts["d_v"]["value"])
    dec = workloads.WORKLOADS["swa_decode_bf16"]
    assert dec.T == 1 + facts["mtp_layers"]["value"]
    assert workloads.WORKLOADS["ga_decode_bf16"].P == facts["max_context"]["value"]


# ---------------------------------------------------------------- planted mistakes must be caught

def _run_pins(mod):
    """Return the list of pins that fail for the oracle-like module ``mod``."""
    failed = []
    s4 = rand(4)
    checks = {
        "bruteforce": lambda: brute_force_err(mod, 1, 6, 4, 2, 3, 2, 3, s4, 0.7) < 1e-13,
        "sdpa": lambda: sdpa_extra_key_err(mod, 1, 12, 4, 2, 8, 5, 4, s4, 0.25) < 1e-12,
        "causal": lambda: causal_sdpa_err(mod, 1, 9, 4, 2, 6, 3, None, 0.3) < 1e-12,
        "window1": lambda: window1_err(mod, 7, 4, 2, 5, 3, s4, 0.4) < 1e-13,
        "decode": lambda: decode_tail_err(mod, 130, 3, 77, 128, 128) < 1e-12,
    }
    for name, fn in checks.items():
        try:
            ok = fn()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    return failed


def test_pins_pass_on_the_oracle():
    assert _run_pins(oracle) == []


def test_planted_dropped_sink_is_caught(monkeypatch):
    orig = oa.sink_attention
    monkeypatch.setattr(oa, "sink_attention", lambda q, qp, k, kp, v, s, sc, w: orig(q, qp, k, kp, v, -np.inf, sc, w))
    assert "sdpa" in _run_pins(oa) and "window1" in _run_pins(oa)


def test_planted_scaled_sink_is_caught(monkeypatch):
    orig = oa.sink_attention
    monkeypatch.setattr(oa, "sink_attention", lambda q, qp, k, kp, v, s, sc, w: orig(q, qp, k, kp, v, s * sc, sc, w))
    assert "sdpa" in _run_pins(oa)


def test_planted_window_off_by_one_is_caught(monkeypatch):
    def vis(q_pos, k_pos, window):
        d = q_pos[:, None] - k_pos[None, :]
        return (d >= 0) & (d <= window)

    monkeypatch.setattr(oa, "visible", vis)
    failed = _run_pins(oa)
    assert "bruteforce" in failed and "window1" in failed


def test_planted_wrong_gqa_map_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "default_kv_map", lambda Hq, Hkv: np.arange(Hq) % Hkv)
    failed = _run_pins(oa)
    assert "causal" in failed and "sdpa" in failed


def test_planted_ring_direction_is_caught(monkeypatch):
    orig = oa.decode_keys

    def wrong(k_new, v_new, k_cache, v_cache, b, P, off, window, T):
        return orig(k_new, v_new, k_cache, v_cache, b, P, -off, window, T)

    monkeypatch.setattr(oa, "decode_keys", wrong)
    assert "decode" in _run_pins(oa)


def test_planted_transposed_value_is_caught(monkeypatch):
    orig = oa.sink_attention

    def wrong(q, qp, k, kp, v, s, sc, w):
        o, lse, lr = orig(q, qp, k, kp, v, s, sc, w)
        return o[::-1].copy(), lse, lr  # rows swapped

    monkeypatch.setattr(oa, "sink_attention", wrong)
    assert "bruteforce" in _run_pins(oa)
