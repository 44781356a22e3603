"""GPU parity: the HIP library (through the C ABI) against the float64 oracle on seeded inputs.

Sizes are small enough for the oracle to finish in seconds but span several tiles and ragged tails;
edge cases cover windows around the tile sizes, single tokens, group sizes 1..16, head maps,
no / -inf / dominant sinks, ring wrap-around, partial rings, every draft count and forced splits.
"""

import numpy as np
import pytest

import oracle
import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd.inputs import decode_inputs, normal, prefill_inputs

from _parity import (assert_lse_close, assert_output_close, f, gpu_from_numpy, say, to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def run_prefill(inp, kv_map=None, window=None, sink=None, use_sink=True):
    dt = inp.dtype
    q, k, v = (gpu_from_numpy(x, dt) for x in (inp.q, inp.k, inp.v))
    s = sink if sink is not None else inp.sink
    s_gpu = torch.from_numpy(np.asarray(s, dtype=np.float32)).cuda() if (use_sink and s is not None) else None
    w = inp.window if window is None else window
    o, lse = mimo.prefill(q, k, v, w, sink=s_gpu, scale=inp.scale, kv_map=kv_map, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.prefill(f(inp.q, dt), f(inp.k, dt), f(inp.v, dt), w,
                                    (s if use_sink else None), inp.scale, kv_head_of_q=kv_map)
    return to_f64(o), to_f64(lse), ref_o, ref_lse


def check_prefill(inp, **kw):
    o, lse, ref_o, ref_lse = run_prefill(inp, **kw)
    m = assert_output_close(o, ref_o, inp.dtype)
    assert_lse_close(lse, ref_lse, inp.dtype)
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv,L,W", [
    (64, 8, 300, 128),    # SWA shape, several tiles, ragged tail
    (64, 4, 257, 10**9),  # global shape
    (64, 4, 200, 128),    # SWA window on the global head layout
])
def test_prefill_mimo_shapes(dtype, Hq, Hkv, L, W):
    say(f"prefill {dtype} Hq={Hq} Hkv={Hkv} L={L} W={W}")
    inp = prefill_inputs(11, 2, L, Hq, Hkv, 192, 128, W, dtype)
    check_prefill(inp)


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257])
def test_prefill_lengths(L):
    say(f"prefill bf16 L={L}")
    check_prefill(prefill_inputs(12, 1, L, 16, 2, 192, 128, 128, "bf16"))
    check_prefill(prefill_inputs(12, 1, L, 16, 2, 192, 128, 10**9, "bf16"))


@pytest.mark.parametrize("W", [1, 2, 3, 31, 32, 33, 63, 64, 65, 100, 127, 129, 200])
def test_prefill_windows(W):
    say(f"prefill windows W={W}")
    check_prefill(prefill_inputs(13, 1, 230, 16, 2, 192, 128, W, "bf16"))
    check_prefill(prefill_inputs(13, 1, 150, 8, 1, 192, 128, W, "f32"))


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2), (12, 1), (32, 2), (24, 3), (128, 8)])
def test_prefill_group_sizes(Hq, Hkv):
    say(f"prefill groups {Hq}/{Hkv}")
    check_prefill(prefill_inputs(14, 2, 170, Hq, Hkv, 192, 128, 64, "bf16"))
    check_prefill(prefill_inputs(14, 1, 170, Hq, Hkv, 192, 128, 10**9, "f32"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_sink_variants(dtype):
    inp = prefill_inputs(15, 1, 160, 16, 2, 192, 128, 128, dtype)
    say("prefill no sink")
    check_prefill(inp, use_sink=False)
    say("prefill -inf sinks")
    check_prefill(inp, sink=np.full(16, -np.inf, np.float32))
    say("prefill mixed sinks")
    mixed = np.array([-np.inf, 0, 3, -3, 8, -20, 1, 2, 40, -np.inf, 0.5, 5, -1, 12, 0, 7], np.float32)
    check_prefill(inp, sink=mixed)
    say("prefill dominant sinks")
    o, lse, ref_o, ref_lse = run_prefill(inp, sink=np.full(16, 1e4, np.float32))
    assert np.all(o == 0.0)
    np.testing.assert_allclose(lse, 1e4, rtol=1e-6)


def test_prefill_global_sink_variants():
    # the global-attention kernel seeds its running max from the sink like the ring kernel does
    inp = prefill_inputs(17, 1, 190, 16, 2, 192, 128, 10**9, "bf16")
    say("global prefill no sink")
    check_prefill(inp, use_sink=False)
    say("global prefill mixed sinks")
    mixed = np.array([-np.inf, 0, 3, -3, 8, -20, 1, 2, 40, -np.inf, 0.5, 5, -1, 12, 0, 7], np.float32)
    check_prefill(inp, sink=mixed)
    say("global prefill dominant sinks")
    o, lse, ref_o, ref_lse = run_prefill(inp, sink=np.full(16, 1e4, np.float32))
    assert np.all(o == 0.0)
    np.testing.assert_allclose(lse, 1e4, rtol=1e-6)


def test_prefill_peaky_scores():
    say("prefill peaky")
    inp = prefill_inputs(16, 1, 200, 16, 2, 192, 128, 128, "bf16")
    inp.q = normal(16, "q", inp.q.shape, "f32") * 8.0
    from sliding_window_sink_seeded_amd.inputs import _f32_to_bf16_bits
    inp.q = _f32_to_bf16_bits(inp.q)
    check_prefill(inp)


def test_prefill_head_map():
    say("prefill explicit head map")
    inp = prefill_inputs(17, 1, 140, 8, 2, 192, 128, 100, "bf16")
    kv_map = [1, 0, 1, 0, 0, 1, 1, 0]
    check_prefill(inp, kv_map=kv_map)


def test_prefill_deterministic():
    say("prefill determinism")
    inp = prefill_inputs(18, 2, 300, 64, 8, 192, 128, 128, "bf16")
    q, k, v = (gpu_from_numpy(x, "bf16") for x in (inp.q, inp.k, inp.v))
    s = torch.from_numpy(inp.sink).cuda()
    o1, l1 = mimo.prefill(q, k, v, 128, sink=s, return_lse=True)
    o2, l2 = mimo.prefill(q, k, v, 128, sink=s, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------------------------- decode

def run_decode(inp, max_len, num_splits=0, kv_map=None, use_offset=True):
    dt = inp.dtype
    g = lambda x: gpu_from_numpy(x, dt)
    lens = torch.from_numpy(inp.cache_len).cuda()
    offs = torch.from_numpy(inp.cache_offset).cuda() if (use_offset and inp.cache_offset is not None) else None
    sink = torch.from_numpy(inp.sink).cuda() if inp.sink is not None else None
    o, lse = mimo.decode(g(inp.q), g(inp.k_new), g(inp.v_new), g(inp.k_cache), g(inp.v_cache), lens,
                         inp.window, max_len, cache_offset=offs, sink=sink, scale=inp.scale,
                         kv_map=kv_map, num_splits=num_splits, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.decode(f(inp.q, dt), f(inp.k_new, dt), f(inp.v_new, dt), f(inp.k_cache, dt),
                                   f(inp.v_cache, dt), inp.cache_len,
                                   inp.cache_offset if use_offset else None, inp.window, inp.sink,
                                   inp.scale, kv_head_of_q=kv_map)
    return to_f64(o), to_f64(lse), ref_o, ref_lse


def check_decode(inp, max_len, **kw):
    o, lse, ref_o, ref_lse = run_decode(inp, max_len, **kw)
    assert_output_close(o, ref_o, inp.dtype)
    assert_lse_close(lse, ref_lse, inp.dtype)
    return o


RING_LENS = np.array([0, 1, 2, 5, 31, 32, 33, 100, 126, 127, 128, 129, 200, 1000, 4097, 32767],
                     dtype=np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_swa_ring(dtype, T):
    say(f"decode ring {dtype} T={T}")
    inp = decode_inputs(21 + T, len(RING_LENS), T, 64, 8, 192, 128, 128, 128, dtype,
                        len_range=(0, 1))
    inp.cache_len = RING_LENS.copy()
    check_decode(inp, int(RING_LENS.max()))


def test_decode_ring_every_offset():
    say("decode ring offsets 0..127")
    B = 128
    inp = decode_inputs(31, B, 4, 16, 2, 192, 128, 128, 128, "bf16", len_range=(0, 1))
    inp.cache_len = np.full(B, 300, np.int32)
    inp.cache_offset = np.arange(B, dtype=np.int32)
    check_decode(inp, 300)


def test_decode_small_ring():
    say("decode ring C = W - 1")
    inp = decode_inputs(32, 6, 3, 16, 2, 192, 128, 7, 8, "bf16", len_range=(0, 1))
    inp.cache_len = np.array([0, 1, 6, 7, 8, 50], np.int32)
    check_decode(inp, 50)


@pytest.mark.parametrize("T,Hq,Hkv", [(1, 64, 8), (2, 16, 1), (3, 64, 8), (4, 64, 8), (4, 12, 3)])
def test_decode_window_129(T, Hq, Hkv):
    # window 129: 128 committed keys, four full 32-key blocks in one pass; 12/3 heads x 4 tokens
    # leaves 16 of the 32 query columns as padding
    say(f"decode window 129 T={T} {Hq}/{Hkv}")
    lens = np.array([0, 1, 31, 96, 97, 127, 128, 129, 130, 5000], np.int32)
    inp = decode_inputs(35 + T, len(lens), T, Hq, Hkv, 192, 128, 140, 129, "bf16", len_range=(0, 1))
    inp.cache_len = lens
    check_decode(inp, int(lens.max()))


@pytest.mark.parametrize("T", [1, 4])
def test_decode_global_short_cache(T):
    # a global layer whose linear cache holds at most 128 tokens runs the one-pass window kernel
    say(f"decode global, cache <= 128, T={T}")
    inp = decode_inputs(36 + T, 4, T, 64, 8, 192, 128, 128, 10**9, "bf16", ring_offsets=False,
                        len_range=(0, 1))
    inp.cache_len = np.array([0, 17, 100, 128], np.int32)
    check_decode(inp, 128)


@pytest.mark.parametrize("B,Hq,Hkv,T", [(4, 64, 4, 4), (3, 64, 4, 4), (3, 64, 4, 2), (3, 24, 3, 8), (2, 64, 8, 8)])
def test_decode_window_column_chunks(B, Hq, Hkv, T):
    # more than 32 query columns per KV head in one pass: 32-column chunks of the one-pass window
    # kernel, remapped onto one XCD when the (sequence, KV head) pairs come in whole eights
    # (B*Hkv = 16, 16) and in launch order otherwise (12, 9)
    say(f"decode window chunks B={B} {Hq}/{Hkv} T={T}")
    lens = np.array([0, 33, 127, 128, 4000][:B] + [300] * max(0, B - 5), np.int32)
    inp = decode_inputs(38 + T + B, B, T, Hq, Hkv, 192, 128, 128, 128, "bf16", len_range=(0, 1))
    inp.cache_len = lens
    check_decode(inp, int(lens.max()))


def test_decode_ring_one_pass_equals_split():
    say("decode ring: one pass vs two splits")
    inp = decode_inputs(37, 6, 4, 64, 8, 192, 128, 128, 128, "bf16", len_range=(0, 3000))
    one = run_decode(inp, 3000, num_splits=1)
    two = run_decode(inp, 3000, num_splits=2)
    for o in (one, two):
        assert_output_close(o[0], o[2], "bf16")
    assert np.abs(one[0] - two[0]).max() <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("num_splits", [1, 2, 7, 0])
def test_decode_global_splits(dtype, num_splits):
    say(f"decode global {dtype} splits={num_splits}")
    inp = decode_inputs(41, 3, 4, 64, 4, 192, 128, 2100, 10**9, dtype, ring_offsets=False,
                        len_range=(0, 1))
    inp.cache_len = np.array([0, 37, 2100], np.int32)
    check_decode(inp, 2100, num_splits=num_splits)


@pytest.mark.parametrize("T,num_splits", [(8, 1), (8, 2), (8, 7), (8, 0), (5, 0), (5, 3)])
def test_decode_many_columns(T, num_splits):
    # 16 heads x 5..8 tokens = 80..128 query columns per KV head: the column-split kernel (one
    # workgroup of four 32-column waves sharing each staged K/V block); with T = 5 the last 48
    # columns are padding. Lengths: empty, inside the first block, ragged, a full cache.
    say(f"decode many columns T={T} splits={num_splits}")
    inp = decode_inputs(51 + T + num_splits, 4, T, 64, 4, 192, 128, 2100, 10**9, "bf16",
                        ring_offsets=False, len_range=(0, 1))
    inp.cache_len = np.array([0, 17, 1333, 2100], np.int32)
    check_decode(inp, 2100, num_splits=num_splits)


@pytest.mark.parametrize("num_splits", [1, 3, 0])
def test_decode_many_columns_ring(num_splits):
    # the same kernel over a ring of 1000 slots (window 1000) at every kind of offset: the keys of a
    # block wrap around the end of the ring
    say(f"decode many columns, ring, splits={num_splits}")
    inp = decode_inputs(58 + num_splits, 6, 8, 32, 2, 192, 128, 1000, 1000, "bf16", len_range=(0, 1))
    inp.cache_len = np.array([0, 40, 999, 1000, 1017, 4321], np.int32)
    check_decode(inp, 4321, num_splits=num_splits)


def test_decode_split_results_agree():
    say("decode split agreement")
    inp = decode_inputs(42, 2, 4, 64, 4, 192, 128, 5000, 10**9, "bf16", ring_offsets=False,
                        len_range=(0, 1))
    inp.cache_len = np.array([4999, 3333], np.int32)
    outs = [run_decode(inp, 5000, num_splits=n)[0] for n in (1, 2, 7, 0)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-2


def test_decode_offsets_none_equals_zero():
    say("decode offset None == 0")
    inp = decode_inputs(43, 4, 2, 16, 2, 192, 128, 128, 128, "bf16", len_range=(100, 400))
    inp.cache_offset = np.zeros(4, np.int32)
    a = run_decode(inp, 400)[0]
    b = run_decode(inp, 400, use_offset=False)[0]
    assert np.array_equal(a, b)


def test_decode_head_map_and_no_sink():
    say("decode head map, no sink")
    inp = decode_inputs(44, 5, 4, 8, 2, 192, 128, 128, 128, "bf16", len_range=(0, 600),
                        with_sink=False)
    check_decode(inp, 600, kv_map=[1, 1, 0, 0, 1, 0, 1, 0])


def test_decode_deterministic():
    say("decode determinism")
    inp = decode_inputs(45, 2, 4, 64, 4, 192, 128, 3000, 10**9, "bf16", ring_offsets=False,
                        len_range=(2000, 3000))
    a = run_decode(inp, 3000, num_splits=5)[0]
    b = run_decode(inp, 3000, num_splits=5)[0]
    assert np.array_equal(a, b)
