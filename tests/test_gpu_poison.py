"""Parity with every kernel's LDS filled with NaN before it starts (libmimo_attn_poison.so, built
next to the product library with MIMO_POISON_LDS=1; see poison_lds in csrc/common.hpp).

A kernel that reads LDS it has not written in this workgroup - a missing store, padding that is
read and multiplied by zero, a read that overtakes its write behind a missing barrier - produces
NaN here instead of quietly reusing what an earlier workgroup left in LDS. The cases cover every
kernel that uses LDS (each prefill kernel and dtype, the three decode kernels with and without
new-token extensions and splits, both RoPE paths, both backward kernels and the sink reduction),
at small shapes with ragged tails; each is compared with the oracle at the method's tolerances.
"""

import numpy as np
import pytest
import torch

import sliding_window_sink_seeded_amd as mimo
from sliding_window_sink_seeded_amd import build
from sliding_window_sink_seeded_amd.inputs import decode_inputs, output_grad, prefill_inputs

from _parity import assert_output_close, say
from test_gpu_backward import check_all
from test_gpu_parity import check_decode, check_prefill
from test_gpu_rope import BASES, check_lse, run_decode_rope, run_prefill_rope

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def poisoned_library():
    saved_lib, saved_path = mimo._lib, mimo.LIB_PATH
    mimo._lib, mimo.LIB_PATH = None, build.LIB_POISON
    try:
        lib = mimo.library()  # raises if the checking library is not built
        assert lib._name == build.LIB_POISON, lib._name
        yield
    finally:
        torch.cuda.synchronize()
        mimo._lib, mimo.LIB_PATH = saved_lib, saved_path


@pytest.mark.parametrize("dtype,Hq,Hkv,L,W", [
    ("bf16", 64, 8, 300, 128),      # sliding-window ring kernel
    ("bf16", 16, 2, 257, 10**9),    # global ping-pong kernel
    ("bf16", 16, 4, 230, 64),       # generic kernel, 32-key blocks
    ("bf16", 64, 8, 190, 200),      # generic kernel, 64-key blocks
    ("f32", 8, 1, 150, 10**9),      # fp32 kernel
    ("f32", 64, 8, 200, 128),
])
def test_poisoned_prefill(dtype, Hq, Hkv, L, W):
    say(f"poisoned LDS: prefill {dtype} {Hq}/{Hkv} L={L} W={W}")
    check_prefill(prefill_inputs(71, 2, L, Hq, Hkv, 192, 128, W, dtype))


@pytest.mark.parametrize("dtype,T,Hq,Hkv,C,W,lens,splits", [
    ("bf16", 4, 64, 8, 128, 128, [0, 5, 127, 128, 3000], 0),        # window kernel, 32 columns
    ("bf16", 8, 64, 8, 128, 128, [0, 5, 127, 128, 3000], 0),        # window kernel, 64 columns, 8 tokens
    ("bf16", 2, 64, 8, 700, 10**9, [0, 33, 500, 700], 3),           # decode_kernel, 16 columns, splits
    ("bf16", 4, 64, 4, 1500, 10**9, [0, 33, 1000, 1500], 0),        # column-split kernel, 64 columns
    ("bf16", 8, 64, 4, 1500, 10**9, [0, 33, 1000, 1500], 1),        # column-split kernel, 128 columns
    ("bf16", 5, 64, 4, 1000, 1000, [0, 40, 999, 4321], 3),          # ring, 80 columns, splits
    ("f32", 4, 64, 4, 700, 10**9, [0, 33, 500, 700], 2),            # fp32, column chunks
])
def test_poisoned_decode(dtype, T, Hq, Hkv, C, W, lens, splits):
    say(f"poisoned LDS: decode {dtype} T={T} {Hq}/{Hkv} C={C} W={W} splits={splits}")
    lens = np.array(lens, np.int32)
    inp = decode_inputs(72 + T, len(lens), T, Hq, Hkv, 192, 128, C, W, dtype,
                        ring_offsets=W < 10**9, len_range=(0, 1))
    inp.cache_len = lens
    check_decode(inp, int(lens.max()), num_splits=splits)


def test_poisoned_rope():
    say("poisoned LDS: RoPE prefill (ring kernel) and decode (window and column-split kernels)")
    inp = prefill_inputs(73, 2, 300, 64, 8, 192, 128, 128, "bf16")
    o, lse, ref_o, ref_lse = run_prefill_rope(inp, BASES["swa"])
    assert_output_close(o, ref_o, "bf16")
    check_lse(lse, ref_lse, "bf16")
    for T, Hkv, C, W, splits in ((4, 8, 128, 128, 0), (8, 4, 700, 10**9, 3)):
        inp = decode_inputs(74 + T, 3, T, 64, Hkv, 192, 128, C, W, "bf16", len_range=(100, C),
                            ring_offsets=W < 10**9)
        o, lse, ref_o, ref_lse = run_decode_rope(inp, C, BASES["swa" if W < 10**9 else "ga"], splits)
        assert_output_close(o, ref_o, "bf16")
        check_lse(lse, ref_lse, "bf16")


@pytest.mark.parametrize("dtype,B,L,Hq,Hkv,W", [
    ("bf16", 2, 300, 64, 8, 128),     # two-wave dK/dV workgroups; the sliding-window dQ walk
    ("bf16", 1, 700, 8, 1, 64),       # the dQ walk with every block masked, three segments
    ("bf16", 1, 297, 16, 2, 10**9),   # paired key blocks
    ("f32", 1, 150, 8, 1, 10**9),
])
def test_poisoned_backward(dtype, B, L, Hq, Hkv, W):
    say(f"poisoned LDS: backward {dtype} B={B} L={L} {Hq}/{Hkv} W={W}")
    inp = prefill_inputs(75, B, L, Hq, Hkv, 192, 128, W, dtype)
    check_all(inp, output_grad(75, B, L, Hq, 128, dtype))
