"""Seeded sweep over random small shapes: every entry point against the oracle on shapes drawn
from the ranges the ABI accepts (sequence lengths, windows, GQA groups, draft counts, ring sizes
and offsets, both dtypes), so that shape combinations no hand-written case names are covered.
Each case prints its parameters first, so a failure names its shape."""

import numpy as np
import pytest

import oracle
import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd.inputs import decode_inputs, output_grad, prefill_inputs

from _parity import (assert_grad_close, assert_lse_close, assert_output_close, f, gpu_from_numpy, say,
                     to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)

GROUPS = [(8, 8), (16, 8), (16, 2), (64, 8), (64, 4), (12, 3), (6, 1)]


def draw_prefill(seed):
    r = np.random.default_rng(seed)
    Hq, Hkv = GROUPS[r.integers(len(GROUPS))]
    L = int(r.integers(1, 400))
    W = int(r.choice([1, 2, 31, 32, 33, 64, 127, 128, 129, 200, 10**9]))
    B = int(r.integers(1, 3))
    dtype = str(r.choice(["bf16", "f32"]))
    sink = bool(r.integers(0, 4))  # mostly with a sink
    return dict(B=B, L=L, Hq=Hq, Hkv=Hkv, W=W, dtype=dtype, sink=sink)


@pytest.mark.parametrize("seed", range(200, 224))
def test_random_prefill_forward_and_backward(seed):
    c = draw_prefill(seed)
    say(f"random prefill seed={seed} {c}")
    dt = c["dtype"]
    inp = prefill_inputs(seed, c["B"], c["L"], c["Hq"], c["Hkv"], 192, 128, c["W"], dt,
                         with_sink=c["sink"])
    q, k, v = (gpu_from_numpy(x, dt) for x in (inp.q, inp.k, inp.v))
    sink = torch.from_numpy(inp.sink).cuda() if inp.sink is not None else None
    o, lse = mimo.prefill(q, k, v, c["W"], sink=sink, scale=inp.scale, return_lse=True)
    d_o = output_grad(seed, c["B"], c["L"], c["Hq"], 128, dt)
    dq, dk, dv, ds = mimo.prefill_backward(q, k, v, o, lse, gpu_from_numpy(d_o, dt), c["W"], sink=sink,
                                           scale=inp.scale)
    torch.cuda.synchronize()
    args = (f(inp.q, dt), f(inp.k, dt), f(inp.v, dt))
    ref_o, ref_lse = oracle.prefill(*args, c["W"], inp.sink, inp.scale)
    assert_output_close(to_f64(o), ref_o, dt)
    assert_lse_close(to_f64(lse), ref_lse, dt)
    rq, rk, rv, rs = oracle.prefill_backward(*args, f(d_o, dt), c["W"], inp.sink, inp.scale)
    # the method's gradient bars (tests/_parity.py GRAD_TOL). With W = 1 and no sink every row
    # sees only its own key with weight exactly 1, so ds = p (dp - D) = 0 and dq, dk vanish
    # identically: there the check is absolute (the kernels' dp and D are fp32 sums of the same
    # products in different orders, so their difference is rounding-sized, about 1e-5 of dO.v ~ 10
    # times scale).
    degenerate = c["W"] == 1 and inp.sink is None
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g64 = to_f64(got)
        if degenerate and name != "dv":
            assert np.array_equal(ref, np.zeros_like(ref)) and np.abs(g64).max() <= 1e-4, name
            continue
        assert_grad_close(g64, ref, dt, f"seed {seed} {name}")
    assert (ds is None) == (inp.sink is None)


def draw_decode(seed):
    r = np.random.default_rng(seed)
    Hq, Hkv = GROUPS[r.integers(len(GROUPS))]
    T = int(r.integers(1, 9))
    ring = bool(r.integers(0, 2))
    B = int(r.integers(1, 6))
    dtype = str(r.choice(["bf16", "f32"]))
    if ring:
        W = int(r.choice([16, 64, 127, 128, 129]))
        C = int(r.integers(W - 1, W + 40)) if W > 1 else 1
        max_len = int(r.integers(1, 3000))
    else:
        W = 10**9
        max_len = int(r.integers(1, 1500))
        C = max_len + int(r.integers(0, 5))
    splits = int(r.choice([0, 0, 1, 2, 5]))
    return dict(B=B, T=T, Hq=Hq, Hkv=Hkv, W=W, C=C, max_len=max_len, ring=ring, dtype=dtype,
                splits=splits)


@pytest.mark.parametrize("seed", range(300, 324))
def test_random_decode_and_commit(seed):
    c = draw_decode(seed)
    say(f"random decode seed={seed} {c}")
    dt = c["dtype"]
    inp = decode_inputs(seed, c["B"], c["T"], c["Hq"], c["Hkv"], 192, 128, c["C"], c["W"], dt,
                        len_range=(0, c["max_len"] + 1), ring_offsets=c["ring"])
    g = lambda x: gpu_from_numpy(x, dt)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    offs = i32(inp.cache_offset) if inp.cache_offset is not None else None
    kc, vc = g(inp.k_cache), g(inp.v_cache)
    len_t = i32(inp.cache_len)
    kn, vn = g(inp.k_new), g(inp.v_new)
    o, lse = mimo.decode(g(inp.q), kn, vn, kc, vc, len_t, c["W"], c["max_len"], cache_offset=offs,
                         sink=torch.from_numpy(inp.sink).cuda(), scale=inp.scale,
                         num_splits=c["splits"], return_lse=True)
    torch.cuda.synchronize()
    args = (f(inp.q, dt), f(inp.k_new, dt), f(inp.v_new, dt), f(inp.k_cache, dt), f(inp.v_cache, dt))
    ref_o, ref_lse = oracle.decode(*args, inp.cache_len, inp.cache_offset, c["W"], inp.sink, inp.scale)
    assert_output_close(to_f64(o), ref_o, dt)
    assert_lse_close(to_f64(lse), ref_lse, dt)
    # commit a random accepted prefix and compare the caches bit for bit
    acc = np.random.default_rng(seed + 1).integers(0, c["T"] + 1, c["B"]).astype(np.int32)
    cap = c["max_len"] + c["T"] if c["ring"] else c["C"]  # a linear cache holds positions < C
    mimo.cache_append(kn, vn, kc, vc, len_t, cap, cache_offset=offs, accept=i32(acc))
    torch.cuda.synchronize()
    eff = np.minimum(acc, cap - inp.cache_len)
    rk, rv, rl = oracle.cache_append(args[1], args[2], args[3], args[4], inp.cache_len,
                                     inp.cache_offset, eff)
    assert np.array_equal(len_t.cpu().numpy(), rl)
    assert np.array_equal(to_f64(kc), rk.astype(np.float64))
    assert np.array_equal(to_f64(vc), rv.astype(np.float64))
