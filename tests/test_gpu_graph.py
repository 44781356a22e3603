"""The entry points under HIP graph capture (torch.cuda.CUDAGraph on the caller's stream).

None of them allocates, synchronises or clears memory with a memset: everything they launch can be
recorded once and replayed. Each test captures once, then replays several times with new inputs
copied into the captured buffers by ordinary eager work, synchronising between replays, and checks
every replay bit for bit against the same call made eagerly on the same data, and against the
oracle:

* a serving step (verify T drafts of every sequence, then commit the accepted prefix) captured
  once and replayed until every sequence has been fed in full; cache_len advances on the device, so
  each replay reads the lengths the previous one left;
* prefill and its backward captured together and replayed on three seeded inputs.
"""

import numpy as np
import pytest

import oracle
import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd.inputs import normal, output_grad, prefill_inputs

from _parity import (SINK_TOL, assert_grad_close, assert_lse_close, assert_output_close, f, gpu_from_numpy,
                     say, sink_grad_rel_err, to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


@pytest.mark.parametrize("layer,T", [("swa", 4), ("swa", 8), ("ga", 4)])
def test_graph_verify_commit_loop(layer, T):
    say(f"graph verify/commit loop {layer} T={T}")
    dt, B, N = "bf16", 3, 300
    Hq, Hkv, W = (64, 8, 128) if layer == "swa" else (64, 4, 10**9)
    C = 128 if layer == "swa" else N
    seq = prefill_inputs(140 + T, B, N, Hq, Hkv, 192, 128, W, dt)
    ref, _ = oracle.prefill(f(seq.q, dt), f(seq.k, dt), f(seq.v, dt), W, seq.sink, seq.scale)
    r = np.random.default_rng(11 + T)
    offs = i32(r.integers(0, C, B)) if layer == "swa" else None
    kc = torch.zeros((B, C, Hkv, 192), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((B, C, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    len_t = i32(np.zeros(B))
    sink = torch.from_numpy(seq.sink).cuda()
    Q, K, V = (gpu_from_numpy(x, dt) for x in (seq.q, seq.k, seq.v))
    # the captured buffers: this step's drafts, accepted counts, output and split workspace
    qn = torch.zeros((B, T, Hq, 192), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((B, T, Hkv, 192), dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros((B, T, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    acc_t = i32(np.zeros(B))
    o_g = torch.empty((B, T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, mimo.decode_workspace_size(B, T, Hq, Hkv, 128, N, W)), dtype=torch.uint8,
                     device="cuda")

    def step(out):
        mimo.decode(qn, kn, vn, kc, vc, len_t, W, N, cache_offset=offs, sink=sink, scale=seq.scale,
                    workspace=ws, out=out)

    def commit():
        mimo.cache_append(kn, vn, kc, vc, len_t, N, cache_offset=offs, accept=acc_t)

    # first launches of every kernel outside the capture (nothing committed: accept = 0)
    step(o_g)
    commit()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(o_g)
        commit()
    torch.cuda.synchronize()
    assert np.array_equal(len_t.cpu().numpy(), np.zeros(B)), "capture must not run the work"

    junk = lambda name, shape: gpu_from_numpy(normal(int(r.integers(1 << 30)), name, shape, dt), dt)
    P = np.zeros(B, np.int64)
    got = [dict() for _ in range(B)]
    replays = 0
    while (P < N).any():
        acc = np.array([min(int(r.integers(1, T + 1)), N - p) for p in P])
        qn.copy_(junk("q", qn.shape))
        kn.copy_(junk("k", kn.shape))
        vn.copy_(junk("v", vn.shape))
        for b in range(B):
            a, p = int(acc[b]), int(P[b])
            qn[b, :a], kn[b, :a], vn[b, :a] = Q[b, p:p + a], K[b, p:p + a], V[b, p:p + a]
        acc_t.copy_(i32(acc))
        o_e = torch.empty_like(o_g)
        step(o_e)  # the eager call on the same cache state
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {replays} differs from the eager call"
        assert np.array_equal(len_t.cpu().numpy(), P + acc)
        o = to_f64(o_g)
        for b in range(B):
            for t in range(int(acc[b])):
                got[b][int(P[b]) + t] = o[b, t]
        P += acc
        replays += 1
    say(f"    {replays} replays")
    out = np.stack([np.stack([got[b][i] for i in range(N)]) for b in range(B)])
    assert_output_close(out, ref, dt)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("W,Hq,Hkv", [(128, 16, 2), (10**9, 32, 2)])
def test_graph_prefill_and_backward(dtype, W, Hq, Hkv):
    say(f"graph prefill+backward {dtype} W={W} Hq={Hq} Hkv={Hkv}")
    B, L = 2, 197
    first = prefill_inputs(160, B, L, Hq, Hkv, 192, 128, W, dtype)
    q, k, v = (gpu_from_numpy(x, dtype) for x in (first.q, first.k, first.v))
    d_o = gpu_from_numpy(output_grad(160, B, L, Hq, 128, dtype), dtype)
    sink = torch.from_numpy(first.sink).cuda()
    o = torch.empty((B, L, Hq, 128), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(mimo.backward_workspace_size(B, L, Hq), dtype=torch.uint8, device="cuda")
    dsink_box = []

    def run(o_, lse_, grads_):
        mimo.prefill(q, k, v, W, sink=sink, scale=first.scale, out=o_, lse=lse_)
        res = mimo.prefill_backward(q, k, v, o_, lse_, d_o, W, sink=sink, scale=first.scale,
                                    workspace=ws, out=grads_)
        return res[3]

    run(o, lse, grads)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dsink_box.append(run(o, lse, grads))
    dsink_g = dsink_box[0]
    for seed in (161, 162, 163):
        inp = prefill_inputs(seed, B, L, Hq, Hkv, 192, 128, W, dtype)
        dO = output_grad(seed, B, L, Hq, 128, dtype)
        for dst, src in ((q, inp.q), (k, inp.k), (v, inp.v), (d_o, dO)):
            dst.copy_(gpu_from_numpy(src, dtype))
        sink.copy_(torch.from_numpy(inp.sink))
        o_e, lse_e = torch.empty_like(o), torch.empty_like(lse)
        grads_e = tuple(torch.empty_like(t) for t in grads)
        dsink_e = run(o_e, lse_e, grads_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, e in (("o", o, o_e), ("lse", lse, lse_e), ("dq", grads[0], grads_e[0]),
                           ("dk", grads[1], grads_e[1]), ("dv", grads[2], grads_e[2]),
                           ("dsink", dsink_g, dsink_e)):
            assert torch.equal(a, e), f"seed {seed}: replayed {name} differs from the eager call"
        args = (f(inp.q, dtype), f(inp.k, dtype), f(inp.v, dtype))
        ref_o, ref_lse = oracle.prefill(*args, W, inp.sink, inp.scale)
        assert_output_close(to_f64(o), ref_o, dtype)
        assert_lse_close(to_f64(lse), ref_lse, dtype)
        rq, rk, rv, rs = oracle.prefill_backward(*args, f(dO, dtype), W, inp.sink, inp.scale)
        # the method's gradient bars (tests/_parity.py GRAD_TOL, SINK_TOL)
        for name, got, ref in (("dq", grads[0], rq), ("dk", grads[1], rk), ("dv", grads[2], rv)):
            assert_grad_close(to_f64(got), ref, dtype, f"seed {seed} {name}")
        err = sink_grad_rel_err(dsink_g.cpu().numpy(), rs, f(dO, dtype), ref_o, ref_lse, inp.sink)
        assert err.max() <= SINK_TOL[dtype], (seed, "dsink", err.max())
