"""The streamed whole-tensor comparison (tests/_fullsize.py) checked on the CPU: fed the oracle's own
whole-tensor result it must report zero error, and fed a result with one planted error it must
report exactly that error - so its unit slicing (key halos, RoPE positions, head groups, ring
offsets) covers every element once and loses nothing."""

import types

import numpy as np
import pytest

import oracle
from sliding_window_sink_seeded_amd.inputs import as_float, decode_inputs, prefill_inputs

import _fullsize

torch = pytest.importorskip("torch")


def wl(**kw):
    base = dict(dtype="bf16", dqk=192, dv=128, rope_base=0.0)
    base.update(kw)
    return types.SimpleNamespace(**base)


def as_torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("rope", [0.0, 1e4])
def test_prefill_windowed_covers_every_row(rope):
    w = wl(B=2, L=700, Hq=16, Hkv=2, window=128, rope_base=rope)
    inp = prefill_inputs(5, w.B, w.L, w.Hq, w.Hkv, 192, 128, w.window, "bf16")
    args = [as_float(x, "bf16") for x in (inp.q, inp.k, inp.v)]
    if rope:
        ref, ref_lse = oracle.prefill_rope(*args, w.window, inp.sink, inp.scale, rope)
    else:
        ref, ref_lse = oracle.prefill(*args, w.window, inp.sink, inp.scale)
    o = torch.from_numpy(ref)
    lse = torch.from_numpy(ref_lse)
    m = _fullsize.prefill_windowed(w, inp, o, lse, rows_per_unit=160).metrics()
    assert m["elements"] == ref.size and m["abs_max"] <= 1e-12 and m["lse_abs"] <= 1e-12, m
    bad = ref.copy()
    bad[1, 333, 7, 5] += 0.25  # one planted error in a unit that does not start at row 0
    m = _fullsize.prefill_windowed(w, inp, torch.from_numpy(bad), lse, rows_per_unit=160).metrics()
    assert abs(m["abs_max"] - 0.25) <= 1e-12
    np.testing.assert_allclose(m["rel_l2"], 0.25 / np.linalg.norm(ref), rtol=1e-9)


@pytest.mark.parametrize("rope", [0.0, 5e6])
def test_prefill_rows_global(rope):
    w = wl(B=1, L=300, Hq=8, Hkv=2, window=10**9, rope_base=rope)
    inp = prefill_inputs(6, 1, w.L, w.Hq, w.Hkv, 192, 128, w.window, "bf16")
    args = [as_float(x, "bf16") for x in (inp.q, inp.k, inp.v)]
    if rope:
        ref, ref_lse = oracle.prefill_rope(*args, w.window, inp.sink, inp.scale, rope)
    else:
        ref, ref_lse = oracle.prefill(*args, w.window, inp.sink, inp.scale)
    rows = [(0, i) for i in (0, 1, 63, 64, 255, 299)]
    m = _fullsize.prefill_rows(w, inp, torch.from_numpy(ref), torch.from_numpy(ref_lse), rows).metrics()
    assert m["elements"] == len(rows) * w.Hq * 128 and m["abs_max"] <= 1e-12 and m["lse_abs"] <= 1e-12, m


@pytest.mark.parametrize("rope,ring", [(0.0, True), (1e4, True), (0.0, False), (5e6, False)])
def test_decode_all_covers_every_output(rope, ring):
    B, T, Hq, Hkv = 5, 3, 16, 4
    C, W = (128, 128) if ring else (400, 10**9)
    w = wl(B=B, T=T, Hq=Hq, Hkv=Hkv, window=W, rope_base=rope)
    inp = decode_inputs(7, B, T, Hq, Hkv, 192, 128, C, W, "bf16", len_range=(0, 400),
                        ring_offsets=ring)
    args = [as_float(x, "bf16") for x in (inp.q, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache)]
    rest = (inp.cache_len, inp.cache_offset, W, inp.sink, inp.scale)
    ref, ref_lse = (oracle.decode_rope(*args, *rest, rope) if rope else oracle.decode(*args, *rest))
    m = _fullsize.decode_all(w, inp, torch.from_numpy(ref), torch.from_numpy(ref_lse)).metrics()
    assert m["elements"] == ref.size and m["abs_max"] <= 1e-12 and m["lse_abs"] <= 1e-12, m
    bad = ref.copy()
    bad[4, 2, 13, 100] -= 0.5
    m = _fullsize.decode_all(w, inp, torch.from_numpy(bad), torch.from_numpy(ref_lse)).metrics()
    assert abs(m["abs_max"] - 0.5) <= 1e-12


def test_error_sums_merge_equals_one_pass():
    rng = np.random.default_rng(3)
    got, ref = rng.standard_normal((2, 50, 7))
    whole = _fullsize.ErrorSums().add(got, ref).metrics()
    parts = _fullsize.ErrorSums()
    for i in range(0, 50, 13):
        parts.merge(_fullsize.ErrorSums().add(got[i:i + 13], ref[i:i + 13]))
    m = parts.metrics()
    for key in ("abs_max", "rel_max", "rel_l2"):
        np.testing.assert_allclose(m[key], whole[key], rtol=1e-12)
    d = got - ref
    np.testing.assert_allclose(m["rel_l2"], np.linalg.norm(d) / np.linalg.norm(ref), rtol=1e-12)
