"""GPU parity of cache maintenance and block-draft verification:

* mimo_attn_cache_append against oracle.cache_append, bit for bit (it is a copy), for ring and
  linear caches, accepted counts 0..T and lengths that hit max_cache_len;
* mimo_attn_decode with T = 5..8 new tokens (block drafts) against the oracle, including the
  global layer's 16 heads x 8 tokens = 128 query columns per KV head (two column chunks);
* the verify / commit loop on the device: each step verifies T tokens of which a random prefix
  belongs to the sequence (the rest are junk drafts) and commits that prefix; every accepted
  token's output must equal the oracle's prefill row of the sequence at its position.
"""

import numpy as np
import pytest

import oracle
import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd.inputs import decode_inputs, normal, prefill_inputs

from _parity import assert_output_close, assert_lse_close, f, gpu_from_numpy, say, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 4, 6, 8])
@pytest.mark.parametrize("ring", [True, False])
def test_cache_append_matches_oracle(dtype, T, ring):
    say(f"cache append {dtype} T={T} ring={ring}")
    B, Hkv, C = 6, 4, 128 if ring else 300
    max_len = 10**6 if ring else C
    inp = decode_inputs(90 + T, B, T, 8, Hkv, 192, 128, C, 128, dtype, len_range=(0, 1),
                        ring_offsets=ring)
    lens = np.array([0, 5, 127, 128, 290, 299], np.int32) if not ring else \
        np.array([0, 1, 126, 127, 5000, 99999], np.int32)
    accept = np.array([0, T, 1, T // 2, T, 3 % (T + 1)], np.int32)
    kc, vc = gpu_from_numpy(inp.k_cache, dtype), gpu_from_numpy(inp.v_cache, dtype)
    len_t = i32(lens)
    mimo.cache_append(gpu_from_numpy(inp.k_new, dtype), gpu_from_numpy(inp.v_new, dtype), kc, vc,
                      len_t, max_len, cache_offset=i32(inp.cache_offset) if ring else None,
                      accept=i32(accept))
    torch.cuda.synchronize()
    # the oracle gets the counts the entry point defines: also clamped to max_len - P
    acc_eff = np.minimum(accept, max_len - lens)
    rk, rv, rl = oracle.cache_append(f(inp.k_new, dtype), f(inp.v_new, dtype), f(inp.k_cache, dtype),
                                     f(inp.v_cache, dtype), lens, inp.cache_offset if ring else None,
                                     acc_eff)
    assert np.array_equal(len_t.cpu().numpy(), rl)
    assert np.array_equal(to_f64(kc), rk.astype(np.float64))
    assert np.array_equal(to_f64(vc), rv.astype(np.float64))


def test_cache_append_all_tokens_by_default():
    say("cache append default accept")
    inp = decode_inputs(99, 3, 8, 8, 8, 192, 128, 128, 128, "bf16", len_range=(0, 1000))
    kc, vc = gpu_from_numpy(inp.k_cache, "bf16"), gpu_from_numpy(inp.v_cache, "bf16")
    len_t = i32(inp.cache_len)
    mimo.cache_append(gpu_from_numpy(inp.k_new, "bf16"), gpu_from_numpy(inp.v_new, "bf16"), kc, vc,
                      len_t, 10**6, cache_offset=i32(inp.cache_offset))
    torch.cuda.synchronize()
    rk, _, rl = oracle.cache_append(f(inp.k_new, "bf16"), f(inp.v_new, "bf16"), f(inp.k_cache, "bf16"),
                                    f(inp.v_cache, "bf16"), inp.cache_len, inp.cache_offset, None)
    assert np.array_equal(len_t.cpu().numpy(), rl)
    assert np.array_equal(to_f64(kc), rk.astype(np.float64))


# ----------------------------------------------------------------------- block-draft verification

def run_decode(inp, max_len, num_splits=0):
    dt = inp.dtype
    g = lambda x: gpu_from_numpy(x, dt)
    offs = i32(inp.cache_offset) if inp.cache_offset is not None else None
    o, lse = mimo.decode(g(inp.q), g(inp.k_new), g(inp.v_new), g(inp.k_cache), g(inp.v_cache),
                         i32(inp.cache_len), inp.window, max_len, cache_offset=offs,
                         sink=torch.from_numpy(inp.sink).cuda(), scale=inp.scale,
                         num_splits=num_splits, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.decode(f(inp.q, dt), f(inp.k_new, dt), f(inp.v_new, dt),
                                   f(inp.k_cache, dt), f(inp.v_cache, dt), inp.cache_len,
                                   inp.cache_offset, inp.window, inp.sink, inp.scale)
    assert_output_close(to_f64(o), ref_o, dt)
    assert_lse_close(to_f64(lse), ref_lse, dt)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [5, 6, 8])
def test_ring_decode_block_drafts(dtype, T):
    say(f"ring decode {dtype} T={T}")
    lens = np.array([0, 1, 31, 127, 128, 300, 4097], np.int32)
    inp = decode_inputs(100 + T, len(lens), T, 64, 8, 192, 128, 128, 128, dtype, len_range=(0, 1))
    inp.cache_len = lens
    run_decode(inp, int(lens.max()))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,num_splits", [(6, 0), (8, 0), (8, 1), (8, 3)])
def test_global_decode_block_drafts(dtype, T, num_splits):
    # 16 query heads per KV head x T tokens: 96 or 128 query columns, two column chunks
    say(f"global decode {dtype} T={T} splits={num_splits}")
    inp = decode_inputs(110 + T, 3, T, 64, 4, 192, 128, 900, 10**9, dtype, len_range=(0, 900),
                        ring_offsets=False)
    inp.cache_len[0] = 0
    run_decode(inp, 900, num_splits)


# ------------------------------------------------------------------- the verify / commit loop

@pytest.mark.parametrize("layer,T", [("swa", 4), ("swa", 8), ("ga", 6), ("ga", 8)])
def test_verify_commit_loop(layer, T):
    say(f"verify/commit loop {layer} T={T}")
    dt, B, N = "bf16", 3, 400
    Hq, Hkv, W = (64, 8, 128) if layer == "swa" else (64, 4, 10**9)
    C = 128 if layer == "swa" else N
    seq = prefill_inputs(120 + T, B, N, Hq, Hkv, 192, 128, W, dt)
    ref, _ = oracle.prefill(f(seq.q, dt), f(seq.k, dt), f(seq.v, dt), W, seq.sink, seq.scale)
    r = np.random.default_rng(7 + T)
    offs = r.integers(0, C, B).astype(np.int32) if layer == "swa" else None
    kc = torch.zeros((B, C, Hkv, 192), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((B, C, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    len_t = i32(np.zeros(B))
    off_t = i32(offs) if offs is not None else None
    sink = torch.from_numpy(seq.sink).cuda()
    Q, K, V = (gpu_from_numpy(x, dt) for x in (seq.q, seq.k, seq.v))
    junk = lambda name, shape: gpu_from_numpy(normal(int(r.integers(1 << 30)), name, shape, dt), dt)
    P = np.zeros(B, np.int64)
    got = [dict() for _ in range(B)]
    step = 0
    while (P < N).any():
        acc = np.array([min(int(r.integers(1, T + 1)), N - p) for p in P])  # 0 for finished ones
        qn = junk("q", (B, T, Hq, 192))
        kn = junk("k", (B, T, Hkv, 192))
        vn = junk("v", (B, T, Hkv, 128))
        for b in range(B):
            a, p = int(acc[b]), int(P[b])
            qn[b, :a], kn[b, :a], vn[b, :a] = Q[b, p:p + a], K[b, p:p + a], V[b, p:p + a]
        o, _ = mimo.decode(qn, kn, vn, kc, vc, len_t, W, N, cache_offset=off_t, sink=sink,
                           scale=seq.scale)
        mimo.cache_append(kn, vn, kc, vc, len_t, N, cache_offset=off_t, accept=i32(acc))
        o = to_f64(o)
        for b in range(B):
            for t in range(int(acc[b])):
                got[b][int(P[b]) + t] = o[b, t]
        P += acc
        step += 1
    assert np.array_equal(len_t.cpu().numpy(), np.full(B, N))
    out = np.stack([np.stack([got[b][i] for i in range(N)]) for b in range(B)])
    say(f"    {step} steps")
    assert_output_close(out, ref, dt)
