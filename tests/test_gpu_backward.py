"""GPU parity of the backward pass (mimo_attn_prefill_backward) against the float64 gradient
oracle (oracle/backward.py) on seeded inputs.

The library's forward gives o and lse, the library's backward the gradients (the product path);
the oracle computes the gradients from q, k, v, dO and the sink alone.

Tolerances: the method's bars, applied per gradient (tests/_parity.py GRAD_TOL / SINK_TOL). The
inputs are exactly representable in the storage dtype, so the oracle sees the same values. For
fp32 the kernels stay in fp32 (rounding ~1e-7 per operation, sums of up to a few thousand terms,
measured relative errors <= 2.1e-6). For bf16 the kernels round four quantities to bf16 (relative
error <= 2^-9 = 2.0e-3 each, unbiased): o before D = <dO, o> is formed, p before dV = sum p dO, ds
before dQ and dK, and the outputs themselves; the output rounding alone gives a relative L2 of
about 2^-9 / sqrt(3) = 1.1e-3, and the measured relative L2 errors are 2.3e-3 .. 4.1e-3, inside
the 5e-3 bar.
"""

import numpy as np
import pytest

import oracle
import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd.inputs import output_grad, prefill_inputs

from _parity import (SINK_TOL, assert_grad_close, f, gpu_from_numpy, say, sink_grad_rel_err,
                     to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)

def run(inp, d_o, kv_map=None):
    dt = inp.dtype
    q, k, v = (gpu_from_numpy(x, dt) for x in (inp.q, inp.k, inp.v))
    sink = torch.from_numpy(inp.sink).cuda() if inp.sink is not None else None
    o, lse = mimo.prefill(q, k, v, inp.window, sink=sink, scale=inp.scale, kv_map=kv_map,
                          return_lse=True)
    dq, dk, dv, ds = mimo.prefill_backward(q, k, v, o, lse, gpu_from_numpy(d_o, dt), inp.window,
                                           sink=sink, scale=inp.scale, kv_map=kv_map)
    torch.cuda.synchronize()
    return dict(dq=to_f64(dq), dk=to_f64(dk), dv=to_f64(dv),
                ds=None if ds is None else ds.cpu().numpy().astype(np.float64))


def check_all(inp, d_o, kv_map=None):
    dt = inp.dtype
    got = run(inp, d_o, kv_map)
    args = (f(inp.q, dt), f(inp.k, dt), f(inp.v, dt), f(d_o, dt), inp.window, inp.sink, inp.scale)
    rq, rk, rv, rs = oracle.prefill_backward(*args, kv_head_of_q=kv_map)
    ms = {n: assert_grad_close(got[n], r, dt, n) for n, r in (("dq", rq), ("dk", rk), ("dv", rv))}
    if inp.sink is None:
        assert got["ds"] is None
    else:
        o, lse = oracle.prefill(*args[:3], inp.window, inp.sink, inp.scale, kv_head_of_q=kv_map)
        err = sink_grad_rel_err(got["ds"], rs, args[3], o, lse, inp.sink)
        assert err.max() <= SINK_TOL[dt], f"dsink rel err {err.max()}"
    say("   ", {n: (round(m["rel_l2"], 7), round(m["rel_max"], 7)) for n, m in ms.items()})
    return got


@pytest.mark.parametrize("dtype,B,L,Hq,Hkv,W", [
    ("bf16", 2, 300, 64, 8, 128),      # sliding-window layer shapes
    ("bf16", 2, 257, 16, 2, 10**9),    # global, ragged tail
    ("bf16", 1, 230, 16, 4, 64),
    ("bf16", 1, 161, 64, 4, 10**9),    # global-layer heads, two key blocks, the second partial
    ("f32", 1, 150, 8, 1, 10**9),
    ("f32", 2, 200, 64, 8, 128),
    ("f32", 1, 97, 16, 4, 33),
])
def test_backward_matches_oracle(dtype, B, L, Hq, Hkv, W):
    say(f"backward {dtype} B={B} L={L} {Hq}/{Hkv} W={W}")
    inp = prefill_inputs(60 + L, B, L, Hq, Hkv, 192, 128, W, dtype)
    check_all(inp, output_grad(60 + L, B, L, Hq, 128, dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L,W", [(1, 128), (33, 128), (70, 1), (64, 2), (129, 129)])
def test_backward_edge_shapes(dtype, L, W):
    say(f"backward edge {dtype} L={L} W={W}")
    inp = prefill_inputs(70 + W, 1, L, 8, 2, 192, 128, W, dtype)
    check_all(inp, output_grad(70 + W, 1, L, 8, 128, dtype))


# The sliding-window dQ walk (bf16, window <= 129, 8 or 16 query heads per KV head): one KV head
# and one sequence make the launcher cut the tiles into segments of 8, so these shapes cross
# several segment boundaries (each segment re-reads a 4-block halo), start segments inside the
# first four tiles' zeroed blocks, end on ragged tails, and cover the windows whose middle blocks
# are masked too (W < 128).
@pytest.mark.parametrize("B,L,Hq,Hkv,W", [
    (1, 2100, 8, 1, 128),
    (1, 1000, 16, 1, 129),
    (2, 777, 8, 1, 127),
    (1, 300, 8, 2, 64),
    (1, 40, 8, 1, 1),
    (1, 1, 8, 1, 128),
    (1, 97, 8, 1, 128),
])
def test_backward_sliding_window_segments(B, L, Hq, Hkv, W):
    say(f"backward sliding-window walk B={B} L={L} {Hq}/{Hkv} W={W}")
    inp = prefill_inputs(1000 + L + W, B, L, Hq, Hkv, 192, 128, W, "bf16")
    check_all(inp, output_grad(1000 + L + W, B, L, Hq, 128, "bf16"))


def test_backward_without_sink():
    say("backward no sink")
    inp = prefill_inputs(81, 2, 100, 16, 2, 192, 128, 40, "bf16", with_sink=False)
    check_all(inp, output_grad(81, 2, 100, 16, 128, "bf16"))


def test_backward_explicit_head_map():
    say("backward head map")
    Hq, Hkv = 16, 4
    kv_map = [3, 1, 0, 2, 2, 0, 1, 3, 0, 1, 2, 3, 3, 2, 1, 0]
    inp = prefill_inputs(82, 1, 130, Hq, Hkv, 192, 128, 128, "bf16")
    check_all(inp, output_grad(82, 1, 130, Hq, 128, "bf16"), kv_map=np.array(kv_map))


def test_backward_dominant_sink():
    # a large sink takes almost all of the mass: p is tiny, every gradient is tiny but must still
    # match (relative bars)
    say("backward dominant sink")
    inp = prefill_inputs(83, 1, 90, 8, 1, 192, 128, 50, "f32")
    inp.sink = (inp.sink + 12.0).astype(np.float32)
    check_all(inp, output_grad(83, 1, 90, 8, 128, "f32"))


def test_backward_is_deterministic():
    say("backward determinism")
    inp = prefill_inputs(84, 1, 200, 16, 2, 192, 128, 10**9, "bf16")
    d_o = output_grad(84, 1, 200, 16, 128, "bf16")
    a, b = run(inp, d_o), run(inp, d_o)
    for n in ("dq", "dk", "dv", "ds"):
        assert np.array_equal(a[n], b[n]), n


# ------------------------------------------------------------------ full-size shapes, sampled

def full_size(name, B, L, Hq, Hkv, W, seed, rows, keys):
    say(f"backward full size {name}")
    inp = prefill_inputs(seed, B, L, Hq, Hkv, 192, 128, W, "bf16")
    d_o = output_grad(seed, B, L, Hq, 128, "bf16")
    dt = "bf16"
    q, k, v = (gpu_from_numpy(x, dt) for x in (inp.q, inp.k, inp.v))
    dO = gpu_from_numpy(d_o, dt)
    sink = torch.from_numpy(inp.sink).cuda()
    o, lse = mimo.prefill(q, k, v, W, sink=sink, scale=inp.scale, return_lse=True)
    dq, dk, dv, ds = mimo.prefill_backward(q, k, v, o, lse, dO, W, sink=sink, scale=inp.scale)
    torch.cuda.synchronize()
    say("    kernels done")
    # the oracle reads only the sequences the samples lie in
    for bb in sorted({b for b, _ in rows} | {b for b, _ in keys}):
        args = (f(inp.q[bb:bb + 1], dt), f(inp.k[bb:bb + 1], dt), f(inp.v[bb:bb + 1], dt),
                f(d_o[bb:bb + 1], dt), W, inp.sink, inp.scale)
        r_b = [(0, i) for b, i in rows if b == bb]
        k_b = [(0, j) for b, j in keys if b == bb]
        if r_b:
            ref_q = oracle.backward_rows(*args, r_b)
            got_q = np.stack([to_f64(dq[bb, i]) for _, i in r_b])
            assert_grad_close(got_q, ref_q, dt, f"dq rows of sequence {bb}")
        if k_b:
            ref_k, ref_v = oracle.backward_keys(*args, k_b)
            assert_grad_close(np.stack([to_f64(dk[bb, j]) for _, j in k_b]), ref_k, dt, "dk rows")
            assert_grad_close(np.stack([to_f64(dv[bb, j]) for _, j in k_b]), ref_v, dt, "dv rows")
    say("    sampled rows done")

    # identities at full size, in fp64 on the device, one sequence at a time:
    #   sum q.dq = sum k.dk (bilinear scores), sum v.dv = sum dO.o (output linear in v),
    #   dsink_h = -sum exp(s_h - lse_i) <dO_i, o_i>
    acc = torch.zeros(4, dtype=torch.float64, device="cuda")
    dsum = torch.zeros(Hq, dtype=torch.float64, device="cuda")
    for b in range(B):
        acc[0] += (q[b].double() * dq[b].double()).sum()
        acc[1] += (k[b].double() * dk[b].double()).sum()
        acc[2] += (v[b].double() * dv[b].double()).sum()
        D = (dO[b].double() * o[b].double()).sum(-1)  # [L, Hq]
        acc[3] += D.sum()
        dsum += (torch.exp(sink.double()[None, :] - lse[b].double().T) * D).sum(0)
    a = acc.cpu().numpy()
    # the rounded bf16 outputs bound each identity's error by ~2^-9 of the sum of |terms|
    mag_q = float(sum((q[b].double() * dq[b].double()).abs().sum() for b in range(B)))
    mag_v = float(sum((v[b].double() * dv[b].double()).abs().sum() for b in range(B)))
    assert abs(a[0] - a[1]) <= 1e-2 * mag_q, (a[0], a[1], mag_q)
    assert abs(a[2] - a[3]) <= 1e-2 * mag_v, (a[2], a[3], mag_v)
    np.testing.assert_allclose(ds.double().cpu().numpy(), -dsum.cpu().numpy(), rtol=1e-3, atol=1e-3)


def test_backward_full_size_sliding_window():
    # rows 4095 / 4096 and 28671 / 28672 straddle segments of the sliding-window dQ walk
    rows = [(0, 0), (1, 31), (2, 127), (3, 128), (0, 4095), (0, 4096), (0, 20000), (2, 28671),
            (2, 28672), (3, 32767)]
    keys = [(0, 0), (1, 100), (2, 128), (3, 5000), (0, 32640), (3, 32767)]
    full_size("swa 4 x 32768, 64/8, W=128", 4, 32768, 64, 8, 128, 91, rows, keys)


def test_backward_full_size_global():
    rows = [(0, 0), (0, 1), (0, 4095), (0, 20000), (0, 32767)]
    keys = [(0, 32767), (0, 32740), (0, 32704)]
    full_size("global 1 x 32768, 64/4", 1, 32768, 64, 4, 10**9, 92, rows, keys)
