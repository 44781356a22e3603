"""mimo_attn_decode_noalloc (split partials in the library's static device scratch) against
mimo_attn_decode (partials in a caller workspace), through the C ABI: two calls in a row, the
second smaller, each needing the scratch; then a single-pass call that needs none. Both entry
points run the same kernels with the same split plan, so the outputs must agree bit for bit; each
is also checked against the float64 oracle at the method's bars."""

import pytest

import oracle
import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd.inputs import decode_inputs

from _parity import assert_lse_close, assert_output_close, f, gpu_from_numpy, say, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def both(inp, max_len, nsplit, dtype):
    g = lambda x: gpu_from_numpy(x, dtype)
    B, T, Hq = inp.q.shape[:3]
    args = (g(inp.q), g(inp.k_new), g(inp.v_new), g(inp.k_cache), g(inp.v_cache),
            torch.from_numpy(inp.cache_len).cuda(), inp.window, max_len)
    kw = dict(cache_offset=None if inp.cache_offset is None else torch.from_numpy(inp.cache_offset).cuda(),
              sink=torch.from_numpy(inp.sink).cuda(), scale=inp.scale, num_splits=nsplit)
    outs = {}
    for mode in ("static", None):
        o = torch.empty((B, T, Hq, 128), dtype=args[0].dtype, device="cuda")
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
        outs[mode] = mimo.decode(*args, workspace=mode, out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    return outs["static"], outs[None]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_decode_matches_workspace_decode(dtype):
    cases = [  # (seed, B, T, C, window, max_len, num_splits)
        (61, 5, 4, 3000, 10**9, 3000, 0),   # global cache, automatic plan: 12 splits
        (62, 2, 3, 700, 10**9, 700, 3),     # smaller, over the same scratch: 3 splits
        (63, 3, 4, 128, 128, 5000, 0),      # sliding-window ring: single pass, no partials
    ]
    for seed, B, T, C, W, max_len, nsplit in cases:
        need = mimo.decode_workspace_size(B, T, 64, 4, 128, max_len, W, nsplit)
        say(f"noalloc decode {dtype}: B={B} T={T} C={C} W={W} splits={nsplit} partials={need} bytes")
        assert (need > 0) == (W > max_len)
        inp = decode_inputs(seed, B, T, 64, 4, 192, 128, C, W, dtype, len_range=(1, max_len),
                            ring_offsets=W <= max_len)
        (o_s, l_s), (o_w, l_w) = both(inp, max_len, nsplit, dtype)
        assert torch.equal(o_s, o_w) and torch.equal(l_s, l_w), (
            float((o_s.float() - o_w.float()).abs().max()), float((l_s - l_w).abs().max()))
        ref, ref_lse = oracle.decode(f(inp.q, dtype), f(inp.k_new, dtype), f(inp.v_new, dtype),
                                     f(inp.k_cache, dtype), f(inp.v_cache, dtype), inp.cache_len,
                                     inp.cache_offset, W, inp.sink, inp.scale)
        assert_output_close(to_f64(o_s), ref, dtype)
        assert_lse_close(to_f64(l_s), ref_lse, dtype)
