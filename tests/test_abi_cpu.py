"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, and host
validation rejects bad arguments with the documented codes before anything reaches HIP.

Pointers passed here are fake but aligned addresses: every call below fails validation, so no
device memory is touched.
"""

import ctypes
import os
import re

import pytest

import sliding_window_sink_seeded_amd as mimo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mimo_attn.h")
EINVAL, EUNSUPPORTED, EWORKSPACE = -1, -2, -3
F32, BF16 = 0, 1
P = ctypes.c_void_p(0x10000)  # aligned, never dereferenced
P_MIS = ctypes.c_void_p(0x10008)  # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mimo_attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mimo.LIB_PATH):
        pytest.skip("libmimo_attn.so not built")
    return mimo.library()


def test_header_declares_the_documented_entry_points():
    assert declared_functions() == sorted(mimo.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version(lib):
    assert mimo.version() >= 10000


def prefill(lib, dt=BF16, B=1, L=64, Hq=64, Hkv=8, dqk=192, dv=128, q=P, k=P, v=P, window=128,
            sink=None, kvm=None, scale=0.07, o=P, lse=None):
    return lib.mimo_attn_prefill(dt, B, L, Hq, Hkv, dqk, dv, q, k, v, window, sink, kvm, scale, o,
                                 lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), EUNSUPPORTED),
    (dict(B=0), EINVAL),
    (dict(L=0), EINVAL),
    (dict(Hq=0), EINVAL),
    (dict(Hq=60, Hkv=8), EINVAL),
    (dict(Hq=512, Hkv=8), EUNSUPPORTED),
    (dict(dqk=128), EUNSUPPORTED),
    (dict(dv=192), EUNSUPPORTED),
    (dict(window=0), EINVAL),
    (dict(window=-5), EINVAL),
    (dict(q=None), EINVAL),
    (dict(o=None), EINVAL),
    (dict(k=P_MIS), EINVAL),
    (dict(o=P_MIS), EINVAL),
    (dict(sink=ctypes.c_void_p(0x10002)), EINVAL),
    (dict(lse=ctypes.c_void_p(0x10001)), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(scale=float("inf")), EINVAL),
    (dict(scale=0.0), EINVAL),
    (dict(scale=-0.07), EINVAL),
])
def test_prefill_validation(lib, kw, code):
    assert prefill(lib, **kw) == code
    assert mimo.last_error() != ""


def _kv_map(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return arr, ctypes.cast(arr, ctypes.c_void_p)


@pytest.mark.parametrize("vals", [
    [0, 0, 0, 1],        # KV head 0 serves 3 of the 4 query heads
    [0, 1, 2, 1],        # index out of range for Hkv = 2
    [0, -1, 1, 1],
])
def test_prefill_rejects_bad_head_maps(lib, vals):
    keep, ptr = _kv_map(vals)
    assert prefill(lib, Hq=4, Hkv=2, kvm=ptr) == EINVAL
    assert "kv_head_of_q" in mimo.last_error() or "KV head" in mimo.last_error()


def decode(lib, dt=BF16, B=4, T=4, Hq=64, Hkv=8, dqk=192, dv=128, q=P, kn=P, vn=P, kc=P, vc=P, C=128,
           lens=P, offs=None, max_len=1000, window=128, sink=None, kvm=None, scale=0.07, nsplit=0,
           ws=None, ws_bytes=0, o=P, lse=None):
    return lib.mimo_attn_decode(dt, B, T, Hq, Hkv, dqk, dv, q, kn, vn, kc, vc, C, lens, offs, max_len,
                                window, sink, kvm, scale, nsplit, ws, ws_bytes, o, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), EINVAL),
    (dict(T=9), EINVAL),                      # at most 8 new tokens (block drafts of 6 or 8)
    (dict(C=126), EINVAL),                    # ring too small for W = 128
    (dict(C=0), EINVAL),
    (dict(max_len=-1), EINVAL),
    (dict(nsplit=-1), EINVAL),
    (dict(lens=None), EINVAL),
    (dict(kc=P_MIS), EINVAL),
    (dict(offs=ctypes.c_void_p(0x10002)), EINVAL),
    (dict(dqk=64), EUNSUPPORTED),
    (dict(window=0), EINVAL),
    (dict(scale=0.0), EINVAL),
    (dict(scale=-0.07), EINVAL),
    (dict(window=10**9, C=512, max_len=1000), EINVAL),  # global cache smaller than the history
    (dict(window=10**9, C=1000, max_len=1000, B=2, Hkv=4, Hq=64, nsplit=4), EWORKSPACE),
])
def test_decode_validation(lib, kw, code):
    assert decode(lib, **kw) == code
    assert mimo.last_error() != ""


def decode_noalloc(lib, dt=BF16, B=4, T=4, Hq=64, Hkv=8, dqk=192, dv=128, q=P, kn=P, vn=P, kc=P, vc=P,
                   C=128, lens=P, offs=None, max_len=1000, window=128, sink=None, kvm=None, scale=0.07,
                   nsplit=0, o=P, lse=None):
    return lib.mimo_attn_decode_noalloc(dt, B, T, Hq, Hkv, dqk, dv, q, kn, vn, kc, vc, C, lens, offs,
                                        max_len, window, sink, kvm, scale, nsplit, o, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=9), EINVAL),
    (dict(C=126), EINVAL),
    (dict(lens=None), EINVAL),
    (dict(dqk=64), EUNSUPPORTED),
    (dict(scale=0.0), EINVAL),
    # partials beyond the 64 MiB static scratch: 64 x 4 KV heads x 64 splits x 128 columns x 132
    # floats = 1.1 GB
    (dict(B=64, T=8, Hkv=4, window=10**9, C=262144, max_len=262144, nsplit=64), EWORKSPACE),
])
def test_decode_noalloc_validation(lib, kw, code):
    # the same checks as mimo_attn_decode, all before anything reaches HIP
    assert decode_noalloc(lib, **kw) == code
    assert mimo.last_error() != ""
    if code == EWORKSPACE:
        assert "static decode scratch" in mimo.last_error()


def test_small_ring_is_enough_when_history_is_short(lib):
    # C >= min(W - 1, max_len): with max_len = 100 a 100-slot ring holds every committed key; the
    # call then fails only on the workspace (forced split) - validation of C passed.
    assert decode(lib, C=100, max_len=100, nsplit=2) == EWORKSPACE
    assert decode(lib, C=99, max_len=100, nsplit=2) == EINVAL


def test_workspace_size_query(lib):
    # single pass needs nothing
    assert mimo.decode_workspace_size(256, 4, 64, 8, 128, 32768, 128) == 0
    assert mimo.decode_workspace_size(256, 4, 64, 8, 128, 32768, 128, 1) == 0
    # 8 sequences x 262144 keys, 64/4 heads: 32 splits of 8192 keys, records of 132 floats
    # (128 output values, running max and sum, two pad floats)
    assert mimo.decode_workspace_size(8, 4, 64, 4, 128, 262144, 1 << 30) == 8 * 4 * 32 * 64 * 132 * 4
    assert mimo.decode_workspace_size(8, 4, 64, 4, 128, 262144, 1 << 30, 7) == 8 * 4 * 7 * 64 * 132 * 4
    # invalid arguments -> 0
    assert mimo.decode_workspace_size(8, 9, 64, 4, 128, 1000, 128) == 0
    assert mimo.decode_workspace_size(8, 4, 64, 4, 96, 1000, 128) == 0


def test_binding_fails_loudly_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 2, 192)
    with pytest.raises(ValueError):
        mimo.prefill(x, x[:, :, :1], torch.zeros(1, 4, 1, 128), window=4)


# ------------------------------------------------------------------ rotary-embedding entry points

@pytest.mark.parametrize("n_pos,rot,base,table,code", [
    (0, 64, 1e4, P, EINVAL),
    (100, 64, 1.0, P, EINVAL),
    (100, 64, float("nan"), P, EINVAL),
    (100, 64, float("inf"), P, EINVAL),
    (100, 64, 1e4, None, EINVAL),
    (100, 64, 1e4, P_MIS, EINVAL),
    (100, 32, 1e4, P, EUNSUPPORTED),
])
def test_rope_table_validation(lib, n_pos, rot, base, table, code):
    assert lib.mimo_attn_rope_table(n_pos, rot, base, table, None) == code
    assert mimo.last_error() != ""


def prefill_rope(lib, table=P, positions=64, rot=64, L=64, **kw):
    a = dict(dt=BF16, B=1, Hq=64, Hkv=8, dqk=192, dv=128, q=P, k=P, v=P, window=128, sink=None,
             kvm=None, scale=0.07, o=P, lse=None)
    a.update(kw)
    return lib.mimo_attn_prefill_rope(a["dt"], a["B"], L, a["Hq"], a["Hkv"], a["dqk"], a["dv"],
                                      a["q"], a["k"], a["v"], a["window"], a["sink"], a["kvm"],
                                      a["scale"], table, positions, rot, a.get("ws"), a.get("ws_bytes", 0),
                                      a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), EINVAL),
    (dict(table=P_MIS), EINVAL),
    (dict(positions=63), EINVAL),          # fewer table rows than positions
    (dict(rot=128), EUNSUPPORTED),
    (dict(B=0), EINVAL),                   # the plain prefill checks still apply
    (dict(scale=0.0), EINVAL),
    (dict(ws=P_MIS, ws_bytes=1 << 30, window=10**6), EINVAL),      # misaligned workspace
    (dict(ws=P, ws_bytes=100, window=10**6), EWORKSPACE),           # global layer: too small
])
def test_prefill_rope_validation(lib, kw, code):
    assert prefill_rope(lib, **kw) == code


def decode_rope(lib, table=P, positions=1004, rot=64, max_len=1000, T=4):
    return lib.mimo_attn_decode_rope(BF16, 4, T, 64, 8, 192, 128, P, P, P, P, P, 128, P, None, max_len,
                                     128, None, None, 0.07, table, positions, rot, 0, None, 0,
                                     P, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), EINVAL),
    (dict(positions=1003), EINVAL),        # needs max_len + T rows
    (dict(rot=0), EUNSUPPORTED),
    (dict(T=9, positions=2000), EINVAL),   # the plain decode checks still apply
])
def test_decode_rope_validation(lib, kw, code):
    assert decode_rope(lib, **kw) == code


# ------------------------------------------------------------------------------- backward pass

def backward(lib, dt=BF16, B=1, L=64, Hq=64, Hkv=8, dqk=192, dv=128, lse=P, d_o=P, sink=None,
             dsink=None, dq=P, ws=P, ws_bytes=1 << 30, scale=0.07, window=128, kvm=None):
    return lib.mimo_attn_prefill_backward(dt, B, L, Hq, Hkv, dqk, dv, P, P, P, P, lse, d_o, window,
                                          sink, kvm, scale, dq, P, P, dsink, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), EUNSUPPORTED),
    (dict(L=0), EINVAL),
    (dict(Hq=60), EINVAL),
    (dict(dqk=128), EUNSUPPORTED),
    (dict(window=0), EINVAL),
    (dict(scale=0.0), EINVAL),
    (dict(lse=None), EINVAL),             # the forward's lse is required
    (dict(d_o=None), EINVAL),
    (dict(dq=None), EINVAL),
    (dict(dq=P_MIS), EINVAL),
    (dict(lse=ctypes.c_void_p(0x10002)), EINVAL),
    (dict(dsink=P), EINVAL),              # a sink gradient without a sink
    (dict(ws=None), EINVAL),
    (dict(ws=P_MIS), EINVAL),
    (dict(ws_bytes=100), EWORKSPACE),
])
def test_backward_validation(lib, kw, code):
    assert backward(lib, **kw) == code
    assert mimo.last_error() != ""


def test_backward_workspace_size(lib):
    # D: B * Hq * L floats rounded up to 256 bytes, then Hq * B * ceil(L / 32) sink partials
    assert mimo.backward_workspace_size(2, 100, 8) == 6400 + 8 * 2 * 4 * 4
    assert mimo.backward_workspace_size(1, 33, 3) == 512 + 3 * 1 * 2 * 4
    assert mimo.backward_workspace_size(0, 100, 8) == 0
    # exactly the size query passes the workspace check: the call then fails only on the head map,
    # which is checked after it
    n = mimo.backward_workspace_size(1, 64, 4)
    keep, bad_map = _kv_map([0, 0, 0, 1])
    assert backward(lib, Hq=4, Hkv=2, ws_bytes=n - 1, kvm=bad_map) == EWORKSPACE
    assert backward(lib, Hq=4, Hkv=2, ws_bytes=n, kvm=bad_map) == EINVAL
    assert "KV head" in mimo.last_error()


# ------------------------------------------------------------------------------- cache commit

def append(lib, dt=BF16, B=2, T=4, Hkv=8, dqk=192, dv=128, kn=P, vn=P, kc=P, vc=P, C=128, lens=P,
           offs=None, acc=None, max_len=1000):
    return lib.mimo_attn_cache_append(dt, B, T, Hkv, dqk, dv, kn, vn, kc, vc, C, lens, offs, acc,
                                      max_len, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), EUNSUPPORTED),
    (dict(B=0), EINVAL),
    (dict(T=0), EINVAL),
    (dict(T=9), EINVAL),
    (dict(Hkv=0), EINVAL),
    (dict(dv=192), EUNSUPPORTED),
    (dict(C=0), EINVAL),
    (dict(max_len=-1), EINVAL),
    (dict(lens=None), EINVAL),
    (dict(kc=None), EINVAL),
    (dict(vn=P_MIS), EINVAL),
    (dict(acc=ctypes.c_void_p(0x10002)), EINVAL),
    (dict(offs=ctypes.c_void_p(0x10001)), EINVAL),
])
def test_cache_append_validation(lib, kw, code):
    assert append(lib, **kw) == code
    assert mimo.last_error() != ""


def test_prefill_rope_workspace_size(lib):
    f = lib.mimo_attn_prefill_rope_workspace_size
    f.restype = ctypes.c_size_t
    # bf16 sliding window with 8 query heads per KV head: the ring kernel rotates K once per segment
    assert f(BF16, 4, 32768, 64, 8, 128) == 0
    # the global layer (and fp32, and windows past 129): one rotated copy of K
    assert f(BF16, 1, 32768, 64, 4, 32768) == 1 * 32768 * 4 * 192 * 2
    assert f(BF16, 2, 300, 64, 8, 300) == 2 * 300 * 8 * 192 * 2
    assert f(F32, 1, 512, 64, 8, 128) == 512 * 8 * 192 * 4
    assert f(BF16, 1, 1000, 64, 8, 200) == 1000 * 8 * 192 * 2
    assert f(BF16, 1, 1000, 12, 3, 128) == 1000 * 3 * 192 * 2      # 4 heads per KV head
    assert f(BF16, 0, 10, 8, 8, 10) == 0 and f(BF16, 1, 10, 8, 3, 10) == 0  # invalid shapes
