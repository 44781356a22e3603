"""Full-size parity on the five measured workloads, through the same C-ABI calls the bench times.

The oracle computes sampled output rows one by one (all heads of each sampled row, or a head
subset for the 262144-token global decode); the whole output is additionally checked for
finiteness and run-to-run bitwise determinism. The sliding-window fp32 workload is small enough
for a full-tensor comparison.
"""

import numpy as np
import pytest

import oracle
import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd import inputs, workloads

from _parity import assert_lse_close, assert_output_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def prefill_case(w):
    say(f"workload {w.name}: generating inputs")
    inp = inputs.prefill_inputs(w.seed, w.B, w.L, w.Hq, w.Hkv, w.dqk, w.dv, w.window, w.dtype)
    q, k, v = (inputs.to_torch(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    sink = torch.from_numpy(inp.sink).cuda()
    rope = mimo.rope_table(w.L, w.rope_base) if w.rope_base else None
    say(f"workload {w.name}: launching")
    o1, lse1 = mimo.prefill(q, k, v, w.window, sink=sink, scale=inp.scale, return_lse=True, rope=rope)
    o2, lse2 = mimo.prefill(q, k, v, w.window, sink=sink, scale=inp.scale, return_lse=True, rope=rope)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2), "not deterministic"
    assert bool(torch.isfinite(o1.float()).all()), "non-finite output"
    return inp, o1, lse1


def sampled_prefill_rows(w, inp, o, lse, positions, batches):
    rows = [(b, i) for b in batches for i in positions]
    got = np.stack([o[b, i].float().cpu().numpy() for b, i in rows]).astype(np.float64)
    got_lse = np.stack([lse[b, :, i].cpu().numpy() for b, i in rows]).astype(np.float64)
    ref, ref_lse = [], []
    for b, i in rows:
        lo = max(0, i - w.window + 1)  # row i only reads keys [lo, i]
        rq = np.zeros((1, i - lo + 1, w.Hq, w.dqk), np.float64)
        rq[0, -1] = inputs.as_float(inp.q[b, i], w.dtype)
        rk = inputs.as_float(inp.k[b:b + 1, lo:i + 1], w.dtype).astype(np.float64)
        if w.rope_base:  # rotate by the absolute positions of the slice
            rq[0, -1] = oracle.apply_rope(rq[0, -1][None], [i], w.rope_base)[0]
            rk[0] = oracle.apply_rope(rk[0], np.arange(lo, i + 1), w.rope_base)
        ro, rl = oracle.prefill_rows(rq, rk, inputs.as_float(inp.v[b:b + 1, lo:i + 1], w.dtype),
                                     w.window, inp.sink, inp.scale, [(0, i - lo)])
        ref.append(ro[0]), ref_lse.append(rl[0])
    return got, np.stack(ref), got_lse, np.stack(ref_lse)


def test_swa_prefill_f32_full():
    w = workloads.WORKLOADS["swa_prefill_f32"]
    inp, o, lse = prefill_case(w)
    ref, ref_lse = oracle.prefill(*(inputs.as_float(x, w.dtype) for x in (inp.q, inp.k, inp.v)),
                                  w.window, inp.sink, inp.scale)
    assert_output_close(o.cpu().numpy(), ref, "f32")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "f32")


@pytest.mark.parametrize("name", ["swa_prefill_bf16", "ga_prefill_bf16"])
def test_prefill_workload_sampled(name):
    w = workloads.WORKLOADS[name]
    inp, o, lse = prefill_case(w)
    L = w.L
    positions = sorted({0, 1, 31, 32, 63, 127, 128, 129, 4095, L // 2 + 17, L - 33, L - 2, L - 1})
    if name.startswith("ga"):
        positions = [0, 31, 32, 4096, L // 2 + 17, L - 1]  # late rows read 32K keys each
    say(f"workload {name}: oracle on {len(positions)} positions")
    got, ref, got_lse, ref_lse = sampled_prefill_rows(w, inp, o, lse, positions, sorted({0, w.B - 1}))
    assert_output_close(got, ref, w.dtype)
    check_lse(got_lse, ref_lse, w)


def check_lse(got, ref, w):
    if w.rope_base and w.dtype == "bf16":
        # rotated Q/K are rounded to bf16 in the kernels: see the bound in tests/test_gpu_rope.py
        err = float(np.abs(got - ref).max())
        assert np.isfinite(got).all() and err <= 1e-2, f"lse err {err}"
    else:
        assert_lse_close(got, ref, w.dtype)


@pytest.mark.parametrize("name", ["swa_prefill_rope_bf16", "ga_prefill_rope_bf16"])
def test_prefill_rope_workload_sampled(name):
    test_prefill_workload_sampled(name)


@pytest.mark.parametrize("name", ["swa_decode_bf16", "ga_decode_bf16", "swa_decode_mtp_bf16",
                                  "ga_decode_mtp_bf16", "swa_decode_rope_bf16", "ga_decode_rope_bf16"])
def test_decode_workload_sampled(name):
    w = workloads.WORKLOADS[name]
    say(f"workload {name}: generating inputs")
    inp = inputs.decode_inputs(w.seed, w.B, w.T, w.Hq, w.Hkv, w.dqk, w.dv, w.C, w.window, w.dtype,
                               cache_len=(w.P or None), len_range=(w.len_range or None),
                               ring_offsets=w.ring_offsets)
    t = lambda x: inputs.to_torch(x, w.dtype)
    args = [t(inp.q), t(inp.k_new), t(inp.v_new), t(inp.k_cache), t(inp.v_cache),
            torch.from_numpy(inp.cache_len).cuda()]
    max_len = int(w.P or w.len_range[1])
    kw = dict(cache_offset=(torch.from_numpy(inp.cache_offset).cuda() if inp.cache_offset is not None
                            else None),
              sink=torch.from_numpy(inp.sink).cuda(), scale=inp.scale, return_lse=True)
    if w.rope_base:
        kw["rope"] = mimo.rope_table(max_len + w.T, w.rope_base)
    say(f"workload {name}: launching")
    o1, lse1 = mimo.decode(*args, w.window, max_len, **kw)
    o2, lse2 = mimo.decode(*args, w.window, max_len, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2), "not deterministic"
    assert bool(torch.isfinite(o1.float()).all())
    seqs = [0, 1, w.B - 1]
    heads = list(range(w.Hq)) if name.startswith("swa") or w.P <= 16384 else [0, 5, 17, 31, 40, 63]
    say(f"workload {name}: oracle on sequences {seqs}, {len(heads)} heads")
    sel = lambda x: inputs.as_float(x[seqs], w.dtype)
    dec_args = (sel(inp.q), sel(inp.k_new), sel(inp.v_new), sel(inp.k_cache), sel(inp.v_cache),
                inp.cache_len[seqs], None if inp.cache_offset is None else inp.cache_offset[seqs],
                w.window, inp.sink, inp.scale)
    if w.rope_base:
        ref, ref_lse = oracle.decode_rope(*dec_args, w.rope_base, heads=heads)
    else:
        ref, ref_lse = oracle.decode(*dec_args, heads=heads)
    got = o1[seqs].float().cpu().numpy()[:, :, heads]
    got_lse = lse1[seqs].cpu().numpy()[:, :, heads]
    assert_output_close(got, ref[:, :, heads], w.dtype)
    check_lse(got_lse, ref_lse[:, :, heads], w)
