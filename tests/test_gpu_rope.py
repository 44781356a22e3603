"""GPU parity of the fused partial RoPE paths (rope_table, prefill and decode with unrotated Q/K)
against the float64 oracle (oracle/rope.py) on seeded inputs."""

import numpy as np
import pytest

import oracle
import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd.inputs import decode_inputs, prefill_inputs

from _parity import assert_lse_close, assert_output_close, f, gpu_from_numpy, say, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)

BASES = {"swa": 1e4, "ga": 5e6}  # the pages' bases for sliding-window and global layers

# Output tolerances are the method's (tests/_parity.py). For bf16 the kernels round the rotated
# Q/K values to bf16 before the MFMA, which moves each score by at most
# scale * 2 * 2^-9 * sum over the 64 rotated dims of |q_i k_i| (about 1.2e-2 for N(0,1) entries,
# 1.6e-3 typical); the LSE moves by at most the largest score change of its row, so its bound is
# 1e-2 here instead of the 2e-3 used for unrotated bf16 inputs.
LSE_ABS = {"bf16": 1e-2, "f32": None}


def check_lse(lse, ref_lse, dtype):
    if LSE_ABS[dtype] is None:
        assert_lse_close(lse, ref_lse, dtype)
    else:
        err = float(np.abs(lse - ref_lse).max())
        assert np.isfinite(lse).all() and err <= LSE_ABS[dtype], f"lse err {err}"


@pytest.mark.parametrize("base", [1e4, 6.4e5, 5e6])
def test_rope_table_matches_oracle(base):
    say(f"rope table base={base}")
    n = 40000
    got = mimo.rope_table(n, base).cpu().numpy().astype(np.float64)
    ref = oracle.rope_table(n, base)
    # fp64 evaluation rounded once to fp32: within one fp32 rounding of the exact value
    assert np.abs(got - ref).max() <= 6e-8


def run_prefill_rope(inp, base, window=None):
    dt = inp.dtype
    q, k, v = (gpu_from_numpy(x, dt) for x in (inp.q, inp.k, inp.v))
    s = torch.from_numpy(inp.sink).cuda()
    w = inp.window if window is None else window
    L = inp.q.shape[1]
    table = mimo.rope_table(L + 7, base)
    o, lse = mimo.prefill(q, k, v, w, sink=s, scale=inp.scale, return_lse=True, rope=table)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.prefill_rope(f(inp.q, dt), f(inp.k, dt), f(inp.v, dt), w, inp.sink,
                                         inp.scale, base)
    return to_f64(o), to_f64(lse), ref_o, ref_lse


@pytest.mark.parametrize("dtype,Hq,Hkv,L,W,layer", [
    ("bf16", 64, 8, 300, 128, "swa"),      # sliding-window ring kernel
    ("bf16", 16, 2, 257, 10**9, "ga"),     # global ping-pong kernel (96-key blocks)
    ("bf16", 16, 4, 230, 64, "swa"),       # generic bf16 kernel (32-key blocks)
    ("f32", 8, 1, 150, 10**9, "ga"),       # fp32 kernel
    ("f32", 64, 8, 200, 128, "swa"),
])
def test_prefill_rope(dtype, Hq, Hkv, L, W, layer):
    say(f"prefill rope {dtype} {Hq}/{Hkv} L={L} W={W}")
    inp = prefill_inputs(41, 2, L, Hq, Hkv, 192, 128, W, dtype)
    o, lse, ref_o, ref_lse = run_prefill_rope(inp, BASES[layer])
    assert_output_close(o, ref_o, dtype)
    check_lse(lse, ref_lse, dtype)


@pytest.mark.parametrize("dtype,Hq,Hkv,L,W,layer,same_kernel", [
    ("bf16", 16, 2, 257, 10**9, "ga", False),  # ping-pong (96-key blocks) vs generic (64-key blocks)
    ("bf16", 16, 4, 230, 64, "swa", True),     # generic bf16 kernel (32-key blocks)
    ("bf16", 64, 8, 300, 200, "swa", True),    # a window past the ring kernel's
    ("f32", 8, 1, 150, 10**9, "ga", True),
    ("f32", 64, 8, 200, 128, "swa", True),
])
def test_prefill_rope_k_rotated_once(dtype, Hq, Hkv, L, W, layer, same_kernel):
    # K rotated once into the workspace and K rotated at staging: where one kernel runs both, the
    # same arithmetic on the same values, so the same bits; both against the oracle (the global
    # bf16 layer rotates K once for its ping-pong kernel, whose 96-key blocks sum in another order
    # than the generic kernel that rotates at staging)
    say(f"prefill rope, K rotated once vs at staging: {dtype} {Hq}/{Hkv} L={L} W={W}")
    inp = prefill_inputs(43, 2, L, Hq, Hkv, 192, 128, W, dtype)
    q, k, v = (gpu_from_numpy(x, dtype) for x in (inp.q, inp.k, inp.v))
    s = torch.from_numpy(inp.sink).cuda()
    table = mimo.rope_table(L, BASES[layer])
    need = mimo.prefill_rope_workspace_size(q.dtype, 2, L, Hq, Hkv, W)
    assert need == 2 * L * Hkv * 192 * (2 if dtype == "bf16" else 4)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")  # contents must not matter
    o1, l1 = mimo.prefill(q, k, v, W, sink=s, scale=inp.scale, return_lse=True, rope=table, workspace=ws)
    o2, l2 = mimo.prefill(q, k, v, W, sink=s, scale=inp.scale, return_lse=True, rope=table,
                          rotate_k_once=False)
    torch.cuda.synchronize()
    if same_kernel:
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (
            float((o1.float() - o2.float()).abs().max()), float((l1 - l2).abs().max()))
    ref_o, ref_lse = oracle.prefill_rope(f(inp.q, dtype), f(inp.k, dtype), f(inp.v, dtype), W, inp.sink,
                                         inp.scale, BASES[layer])
    for o, lse in ((o1, l1), (o2, l2)):
        assert_output_close(to_f64(o), ref_o, dtype)
        check_lse(to_f64(lse), ref_lse, dtype)


def test_prefill_rope_changes_the_result():
    # guards against a path that ignores the table: unrotated attention differs from rotated
    inp = prefill_inputs(42, 1, 200, 16, 2, 192, 128, 128, "bf16")
    o, _, ref_o, _ = run_prefill_rope(inp, 1e4)
    plain, _ = oracle.prefill(f(inp.q, "bf16"), f(inp.k, "bf16"), f(inp.v, "bf16"), 128, inp.sink,
                              inp.scale)
    assert np.abs(ref_o - plain).max() > 0.1
    assert_output_close(o, ref_o, "bf16")


def run_decode_rope(inp, max_len, base, num_splits=0):
    dt = inp.dtype
    g = lambda x: gpu_from_numpy(x, dt)
    lens = torch.from_numpy(inp.cache_len).cuda()
    offs = torch.from_numpy(inp.cache_offset).cuda() if inp.cache_offset is not None else None
    sink = torch.from_numpy(inp.sink).cuda()
    T = inp.q.shape[1]
    table = mimo.rope_table(max_len + T, base)
    o, lse = mimo.decode(g(inp.q), g(inp.k_new), g(inp.v_new), g(inp.k_cache), g(inp.v_cache), lens,
                         inp.window, max_len, cache_offset=offs, sink=sink, scale=inp.scale,
                         num_splits=num_splits, return_lse=True, rope=table)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.decode_rope(f(inp.q, dt), f(inp.k_new, dt), f(inp.v_new, dt),
                                        f(inp.k_cache, dt), f(inp.v_cache, dt), inp.cache_len,
                                        inp.cache_offset, inp.window, inp.sink, inp.scale, base)
    return to_f64(o), to_f64(lse), ref_o, ref_lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 4, 5, 8])
def test_decode_rope_ring(dtype, T):
    # T = 5..8: block drafts; new tokens 4..7 take their own staging path in both decode kernels
    say(f"decode rope ring {dtype} T={T}")
    lens = np.array([0, 1, 31, 127, 128, 300, 4097, 32767], np.int32)
    inp = decode_inputs(43 + T, len(lens), T, 64, 8, 192, 128, 128, 128, dtype, len_range=(0, 1))
    inp.cache_len = lens
    o, lse, ref_o, ref_lse = run_decode_rope(inp, int(lens.max()), BASES["swa"])
    assert_output_close(o, ref_o, dtype)
    check_lse(lse, ref_lse, dtype)


@pytest.mark.parametrize("B", [3, 4])
def test_decode_rope_ring_column_chunks(B):
    # 16 query heads per KV head x 4 tokens = 64 columns: the RoPE instance of the one-pass window
    # kernel in 32-column chunks (rotation positions follow each chunk's columns)
    say(f"decode rope ring, column chunks, B={B}")
    lens = np.array([0, 127, 900, 5000][:B], np.int32)
    inp = decode_inputs(49 + B, B, 4, 64, 4, 192, 128, 128, 128, "bf16", len_range=(0, 1))
    inp.cache_len = lens
    o, lse, ref_o, ref_lse = run_decode_rope(inp, int(lens.max()), BASES["swa"])
    assert_output_close(o, ref_o, "bf16")
    check_lse(lse, ref_lse, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("num_splits", [1, 3])
@pytest.mark.parametrize("T", [4, 5, 8])
def test_decode_rope_global(dtype, num_splits, T):
    say(f"decode rope global {dtype} splits={num_splits} T={T}")
    inp = decode_inputs(47 + T, 3, T, 64, 4, 192, 128, 700, 10**9, dtype, len_range=(200, 700),
                        ring_offsets=False)
    o, lse, ref_o, ref_lse = run_decode_rope(inp, 700, BASES["ga"], num_splits)
    assert_output_close(o, ref_o, dtype)
    check_lse(lse, ref_lse, dtype)


def test_decode_rope_continues_a_rope_prefill():
    # rows P..P+T-1 of a RoPE prefill equal a RoPE decode of those tokens whose cache holds the
    # first P keys rotated (here rotated by the oracle) - the position conventions agree
    say("decode rope vs prefill rope")
    B, L, T, Hq, Hkv = 2, 160, 4, 16, 2
    inp = prefill_inputs(48, B, L, Hq, Hkv, 192, 128, 10**9, "f32")
    base = BASES["ga"]
    P = L - T
    q, k, v = (f(x, "f32") for x in (inp.q, inp.k, inp.v))
    kc = np.stack([oracle.apply_rope(k[b, :P], np.arange(P), base) for b in range(B)]).astype(np.float32)
    table = mimo.rope_table(L, base)
    G = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    o_pre, _ = mimo.prefill(G(q), G(k), G(v), 10**9, sink=G(inp.sink), scale=inp.scale, rope=table)
    lens = torch.full((B,), P, dtype=torch.int32, device="cuda")
    o_dec, _ = mimo.decode(G(q[:, P:]), G(k[:, P:]), G(v[:, P:]), G(kc), G(v[:, :P]), lens, 10**9, P,
                           sink=G(inp.sink), scale=inp.scale, rope=table)
    torch.cuda.synchronize()
    assert_output_close(to_f64(o_dec), to_f64(o_pre[:, P:]), "f32")


@pytest.mark.parametrize("rope", [False, True])
def test_ring_prefill_bits_do_not_depend_on_segments(rope):
    # The sliding-window ring kernel cuts each sequence into segments of consecutive tiles whose
    # length follows the grid (batch x KV heads). A tile at a segment start gets its window's key
    # blocks from the segment prologue (with RoPE, rotated there in LDS); mid-segment they arrive one
    # block per tile (rotated as they are staged). Alone, a 8192-token sequence runs in segments of
    # 8 tiles; in a batch of 4, of 32 tiles. Its rows must come out bit for bit the same.
    say(f"ring prefill segment invariance, rope={rope}")
    L, Hq, Hkv, W = 8192, 64, 8, 128
    inp = prefill_inputs(44, 4, L, Hq, Hkv, 192, 128, W, "bf16")
    q, k, v = (gpu_from_numpy(x, "bf16") for x in (inp.q, inp.k, inp.v))
    s = torch.from_numpy(inp.sink).cuda()
    table = mimo.rope_table(L, BASES["swa"]) if rope else None
    o4, l4 = mimo.prefill(q, k, v, W, sink=s, scale=inp.scale, return_lse=True, rope=table)
    o1, l1 = mimo.prefill(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(), W, sink=s,
                          scale=inp.scale, return_lse=True, rope=table)
    torch.cuda.synchronize()
    assert torch.equal(o1[0], o4[0]) and torch.equal(l1[0], l4[0]), (
        float((o1[0].float() - o4[0].float()).abs().max()), float((l1[0] - l4[0]).abs().max()))
