"""Pins for the RoPE oracle (oracle/rope.py), none of which reuses its code path.

* complex form: each rotated pair (x_i, x_{i+32}) is the complex number x_i + j x_{i+32}
  multiplied by exp(j p theta_i) (numpy complex arithmetic, not the cos/sin formula);
* frequencies: theta_0 = 1, consecutive ratios base^(-1/32), theta_31 = base^(-31/32);
* rotation is orthogonal: norms of every pair and of the vector are kept, and the dot product of
  two vectors rotated to the same position is unchanged;
* relative position: <R(m) q, R(n) k> depends on m - n only;
* position 0 is the identity and dimensions 64..191 never change;
* the decode convention (new token t of a sequence with P committed tokens sits at P + t) gives
  the same rows as a prefill over the whole sequence;
* planted mistakes (interleaved pairs, opposite sign, half frequencies, rotating the wrong
  dimensions) each fail at least one of these pins.
"""

import numpy as np
import pytest

import oracle
import oracle.rope as rope_mod


def rng(seed=0):
    return np.random.default_rng(seed)


def complex_rotate(x, positions, base):
    """Independent formulation: pairs as complex numbers times exp(j * p * base^(-2i/64))."""
    x = np.asarray(x, dtype=np.float64)
    z = x[..., :32] + 1j * x[..., 32:64]
    i = np.arange(32)
    theta = base ** (-(2.0 * i) / 64.0)
    p = np.asarray(positions, dtype=np.float64)
    ph = np.exp(1j * np.multiply.outer(p, theta))  # [n, 32]
    if x.ndim == 3:
        ph = ph[:, None, :]
    z = z * ph
    out = x.copy()
    out[..., :32] = z.real
    out[..., 32:64] = z.imag
    return out


def pin_results(mod):
    """Names of the pins that module `mod` (the oracle or a planted mutant) fails."""
    failed = []
    x = rng(1).standard_normal((7, 3, 192))
    pos = np.array([0, 1, 2, 17, 1000, 4095, 262143])
    for base in (10000.0, 5e6):
        y = mod.apply_rope(x, pos, base)
        if not np.allclose(y, complex_rotate(x, pos, base), rtol=1e-12, atol=1e-12):
            failed.append("complex form")
        if not np.array_equal(y[..., 64:], x[..., 64:]):
            failed.append("tail dims unchanged")
        if not np.allclose(y[0], x[0], rtol=0, atol=0):
            failed.append("position 0 identity")
        pair_n0 = x[..., :32] ** 2 + x[..., 32:64] ** 2
        pair_n1 = y[..., :32] ** 2 + y[..., 32:64] ** 2
        if not np.allclose(pair_n0, pair_n1, rtol=1e-12, atol=1e-12):
            failed.append("pair norms")
        # relative position
        q = rng(2).standard_normal(192)
        k = rng(3).standard_normal(192)
        dots = []
        for shift in (0, 5, 1234):
            rq = mod.apply_rope(q[None], [40 + shift], base)[0]
            rk = mod.apply_rope(k[None], [33 + shift], base)[0]
            dots.append(rq @ rk)
        if not np.allclose(dots, dots[0], rtol=1e-10, atol=1e-10):
            failed.append("relative position")
        f = mod.inv_freq(base)
        if not (f[0] == 1.0 and np.allclose(f[1:] / f[:-1], base ** (-1.0 / 32), rtol=1e-13)
                and np.isclose(f[-1], base ** (-31.0 / 32), rtol=1e-13)):
            failed.append("frequencies")
        t = mod.rope_table(5000, base)
        if not (np.allclose(t[..., 0] ** 2 + t[..., 1] ** 2, 1.0, atol=1e-14)
                and np.allclose(t[4095, :, 0] + 1j * t[4095, :, 1],
                                np.exp(1j * 4095 * base ** (-np.arange(32) / 32.0)), atol=1e-12)):
            failed.append("table")
    return sorted(set(failed))


def test_oracle_passes_every_pin():
    assert pin_results(oracle) == []


def test_same_position_keeps_dot_products():
    x = rng(4).standard_normal((5, 192))
    yk = rng(5).standard_normal((5, 192))
    pos = np.array([3, 3, 3, 3, 3])
    a = oracle.apply_rope(x, pos, 1e4)
    b = oracle.apply_rope(yk, pos, 1e4)
    np.testing.assert_allclose(np.sum(a * b, -1), np.sum(x * yk, -1), rtol=1e-12)


def test_decode_positions_match_prefill_rows():
    # a sequence of L tokens: prefill rows L-T..L-1 == decode of the last T tokens with the first
    # P = L - T tokens in a linear cache holding their rotated keys
    r = rng(6)
    B, L, T, Hq, Hkv, W = 1, 50, 3, 4, 2, 1 << 30
    q = r.standard_normal((B, L, Hq, 192))
    k = r.standard_normal((B, L, Hkv, 192))
    v = r.standard_normal((B, L, Hkv, 128))
    sink = r.standard_normal(Hq)
    base, scale = 5e6, 192 ** -0.5
    ref, _ = oracle.prefill_rope(q, k, v, W, sink, scale, base)
    P = L - T
    kc = np.zeros((B, L, Hkv, 192))
    kc[0, :P] = oracle.apply_rope(k[0, :P], np.arange(P), base)
    vc = np.zeros((B, L, Hkv, 128))
    vc[0, :P] = v[0, :P]
    out, _ = oracle.decode_rope(q[:, P:], k[:, P:], v[:, P:], kc, vc, np.array([P]), None, W, sink,
                                scale, base)
    np.testing.assert_allclose(out[0], ref[0, P:], rtol=1e-12, atol=1e-12)


class _Mutant:
    """The oracle module with one function swapped for a planted mistake."""

    def __init__(self, **over):
        self.inv_freq = over.get("inv_freq", rope_mod.inv_freq)
        self.rope_table = over.get("rope_table", rope_mod.rope_table)
        self.apply_rope = over.get("apply_rope", rope_mod.apply_rope)


def _interleaved(x, positions, base, rot_dims=64):
    x = np.array(x, dtype=np.float64, copy=True)
    a = rope_mod.angles(positions, base, rot_dims)
    if x.ndim == 3:
        a = a[:, None, :]
    ev, od = x[..., 0:rot_dims:2].copy(), x[..., 1:rot_dims:2].copy()
    x[..., 0:rot_dims:2] = ev * np.cos(a) - od * np.sin(a)
    x[..., 1:rot_dims:2] = od * np.cos(a) + ev * np.sin(a)
    return x


def _opposite_sign(x, positions, base, rot_dims=64):
    return rope_mod.apply_rope(x, -np.asarray(positions), base, rot_dims)


def _half_freq(base, rot_dims=64):
    return np.power(np.float64(base), -np.arange(rot_dims // 2) / rot_dims)


def _wrong_dims(x, positions, base, rot_dims=64):
    x = np.array(x, dtype=np.float64, copy=True)
    y = rope_mod.apply_rope(x[..., 64:], positions, base, rot_dims)
    x[..., 64:] = y
    return x


@pytest.mark.parametrize("name,mutant", [
    ("interleaved pairs", _Mutant(apply_rope=_interleaved)),
    ("opposite sign", _Mutant(apply_rope=_opposite_sign)),
    ("half frequencies", _Mutant(inv_freq=_half_freq)),
    ("rotates dims 64..127", _Mutant(apply_rope=_wrong_dims)),
])
def test_planted_mistakes_are_caught(name, mutant, monkeypatch):
    if name == "half frequencies":
        # the oracle's angles() reads inv_freq from its module: plant it there
        monkeypatch.setattr(rope_mod, "inv_freq", _half_freq)
        mutant = rope_mod
    assert pin_results(mutant) != [], name
