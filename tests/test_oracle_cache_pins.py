"""Pins for the cache-maintenance oracle (oracle/cache.py).

The pin is the decode loop itself, checked against the prefill oracle (pinned on its own in
test_oracle_pins.py): a stream of tokens is consumed by verify steps of T new tokens, of which
only a random accepted prefix belongs to the stream and the rest are junk drafts; after each step
the accepted prefix is committed with cache_append. Every accepted token's decode output must
equal the prefill row of the stream at its position, whatever the ring size, offset, window and
T, so a mistake in the slot arithmetic, in which tokens are committed or in the length update
makes a later step read a wrong key. Planted mistakes check that it does.
"""

import numpy as np
import pytest

import oracle
import oracle.cache as oc


def run_loop(append, N, T, window, C, off, seed, Hq=4, Hkv=2, dqk=6, dv=5):
    """Max |decode - prefill| over the accepted tokens of a seeded verify loop."""
    r = np.random.default_rng(seed)
    q = r.standard_normal((1, N, Hq, dqk))
    k = r.standard_normal((1, N, Hkv, dqk))
    v = r.standard_normal((1, N, Hkv, dv))
    sink = r.standard_normal(Hq)
    scale = 0.45
    ref, _ = oracle.prefill(q, k, v, window, sink, scale)
    kc = np.zeros((1, C, Hkv, dqk))
    vc = np.zeros((1, C, Hkv, dv))
    lens = np.array([0])
    offs = None if off is None else np.array([off])
    P, worst = 0, 0.0
    while P < N:
        a = int(r.integers(1, T + 1))
        a = min(a, N - P)
        junk = lambda shape: r.standard_normal(shape)
        qn = np.concatenate([q[:, P:P + a], junk((1, T - a, Hq, dqk))], axis=1)
        kn = np.concatenate([k[:, P:P + a], junk((1, T - a, Hkv, dqk))], axis=1)
        vn = np.concatenate([v[:, P:P + a], junk((1, T - a, Hkv, dv))], axis=1)
        o, _ = oracle.decode(qn, kn, vn, kc, vc, lens, offs, window, sink, scale)
        worst = max(worst, float(np.abs(o[0, :a] - ref[0, P:P + a]).max()))
        kc, vc, lens = append(kn, vn, kc, vc, lens, offs, np.array([a]))
        P += a
        if int(lens[0]) != P:
            return float("inf")
    return worst


CASES = [
    # (N, T, window, C, off)
    (40, 1, 5, 4, 3),       # ring of exactly W - 1 slots, one token per step
    (60, 4, 9, 8, 5),
    (70, 8, 9, 11, 0),      # T up to 8 (block drafts)
    (50, 6, 16, 16, 7),
    (45, 8, 10**9, 45, None),  # global layer: linear cache of the whole history
]


def all_pins(append):
    return [c for i, c in enumerate(CASES) if run_loop(append, *c, seed=i) > 1e-12]


def test_decode_loop_with_appends_equals_prefill():
    assert all_pins(oc.cache_append) == []


def test_append_none_and_all():
    r = np.random.default_rng(5)
    kn, vn = r.standard_normal((2, 3, 1, 4)), r.standard_normal((2, 3, 1, 2))
    kc, vc = r.standard_normal((2, 5, 1, 4)), r.standard_normal((2, 5, 1, 2))
    lens = np.array([2, 4])
    k2, v2, l2 = oc.cache_append(kn, vn, kc, vc, lens, None, np.array([0, 0]))
    assert np.array_equal(k2, kc) and np.array_equal(v2, vc) and list(l2) == [2, 4]
    k3, v3, l3 = oc.cache_append(kn, vn, kc, vc, lens, np.array([0, 1]), None)
    assert list(l3) == [5, 7]
    np.testing.assert_array_equal(k3[0, 2:5], kn[0])          # positions 2..4, no wrap
    np.testing.assert_array_equal(k3[1, [0, 1, 2]], kn[1])    # positions 4..6 -> slots 0, 1, 2
    np.testing.assert_array_equal(v3[1, 3:5], vc[1, 3:5])     # untouched slots


# ----------------------------------------------------------------------------- planted mistakes

def _commit_all(kn, vn, kc, vc, lens, offs, accept):
    return oc.cache_append(kn, vn, kc, vc, lens, offs, None)


def _wrong_direction(kn, vn, kc, vc, lens, offs, accept):
    kc, vc, lens = np.array(kc), np.array(vc), np.array(lens)
    C = kc.shape[1]
    for b in range(kn.shape[0]):
        off = 0 if offs is None else int(offs[b])
        for t in range(int(accept[b])):
            s = (off - (int(lens[b]) + t)) % C
            kc[b, s], vc[b, s] = kn[b, t], vn[b, t]
        lens[b] += int(accept[b])
    return kc, vc, lens


def _off_by_one(kn, vn, kc, vc, lens, offs, accept):
    shifted = None if offs is None else np.asarray(offs) + 1
    if offs is None:
        shifted = np.ones(kn.shape[0], dtype=np.int64)
    return oc.cache_append(kn, vn, kc, vc, lens, shifted, accept)


@pytest.mark.parametrize("name,fn", [("commits rejected drafts", _commit_all),
                                     ("ring direction", _wrong_direction),
                                     ("slot off by one", _off_by_one)])
def test_planted_mistakes_are_caught(name, fn):
    assert all_pins(fn) != [], name
