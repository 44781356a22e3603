"""Whole-tensor parity of the full-size workloads against the float64 oracle.

The oracle runs over units of the output (row ranges of one sequence for a prefill, one
(sequence, KV head) for a decode) on a thread pool: numpy releases the interpreter lock inside its
BLAS calls and elementwise loops, so the units run in parallel while each holds only its own slice
of the inputs in float64. Every unit returns running error sums; merged, they give the error
metrics over the whole output tensor, exactly as a single comparison of the two tensors would.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from sliding_window_sink_seeded_amd.inputs import as_float


def host_workers() -> int:
    """Worker threads: the cores this process may run on, at most 16 (one GPU's host share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class ErrorSums:
    """Running sums over compared elements: max |d|, sum d^2, max |ref|, sum ref^2, LSE max |d|."""

    def __init__(self):
        self.d2 = 0.0
        self.r2 = 0.0
        self.dmax = 0.0
        self.rmax = 0.0
        self.lse = 0.0
        self.finite = True
        self.n = 0

    def add(self, got, ref, got_lse=None, ref_lse=None):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        d = got - ref
        self.finite &= bool(np.isfinite(got).all())
        self.d2 += float((d * d).sum())
        self.r2 += float((ref * ref).sum())
        self.dmax = max(self.dmax, float(np.abs(d).max()) if d.size else 0.0)
        self.rmax = max(self.rmax, float(np.abs(ref).max()) if ref.size else 0.0)
        self.n += got.size
        if got_lse is not None:
            gl = np.asarray(got_lse, np.float64)
            self.finite &= bool(np.isfinite(gl).all())
            self.lse = max(self.lse, float(np.abs(gl - ref_lse).max()) if gl.size else 0.0)
        return self

    def merge(self, o):
        self.d2 += o.d2
        self.r2 += o.r2
        self.dmax = max(self.dmax, o.dmax)
        self.rmax = max(self.rmax, o.rmax)
        self.lse = max(self.lse, o.lse)
        self.finite &= o.finite
        self.n += o.n
        return self

    def metrics(self) -> dict:
        return dict(abs_max=self.dmax, rel_max=self.dmax / self.rmax if self.rmax > 0 else self.dmax,
                    rel_l2=float(np.sqrt(self.d2 / self.r2)) if self.r2 > 0 else float(np.sqrt(self.d2)),
                    lse_abs=self.lse, finite=self.finite, elements=self.n)


def run_units(fn, units) -> ErrorSums:
    """fn(unit) -> ErrorSums for every unit on the thread pool (one BLAS thread per worker)."""
    from threadpoolctl import threadpool_limits

    total = ErrorSums()
    with threadpool_limits(1), ThreadPoolExecutor(host_workers()) as ex:
        for part in ex.map(fn, units):
            total.merge(part)
    return total


def f64(x, dtype):
    return np.asarray(as_float(x, dtype), dtype=np.float64)


def prefill_windowed(w, inp, o_host, lse_host, rows_per_unit=1024):
    """Every row of a sliding-window prefill. A unit is rows [i0, i1) of one sequence; the oracle
    sees them as the tail of the slice [i0 - W + 1, i1), which holds every key they can see (the
    slice's leading rows are computed and dropped). With RoPE the slice is rotated by its absolute
    positions first. o_host [B, L, Hq, dv] and lse_host [B, Hq, L] are torch CPU tensors."""
    dt, W = w.dtype, w.window

    def fn(unit):
        b, i0, i1 = unit
        lo = max(0, i0 - W + 1)
        q, k, v = (f64(x[b, lo:i1], dt) for x in (inp.q, inp.k, inp.v))
        if w.rope_base:
            pos = np.arange(lo, i1)
            q = oracle.apply_rope(q, pos, w.rope_base)
            k = oracle.apply_rope(k, pos, w.rope_base)
        ro, rl = oracle.prefill(q[None], k[None], v[None], W, inp.sink, inp.scale)
        got = o_host[b, i0:i1].double().numpy()
        got_lse = lse_host[b, :, i0:i1].numpy()
        return ErrorSums().add(got, ro[0, i0 - lo:], got_lse, rl[0, :, i0 - lo:])

    units = [(b, i0, min(w.L, i0 + rows_per_unit)) for b in range(w.B) for i0 in range(0, w.L, rows_per_unit)]
    return run_units(fn, units)


def prefill_rows(w, inp, o_host, lse_host, rows):
    """Selected rows (b, i), every head, of a prefill of any window (global included). K and V of
    each sequence are widened to float64 once (and, with RoPE, K rotated by its absolute
    positions) and shared by that sequence's rows."""
    dt, W = w.dtype, w.window
    kv = {}
    for b in sorted({b for b, _ in rows}):
        k = f64(inp.k[b], dt)
        if w.rope_base:
            k = oracle.apply_rope(k, np.arange(w.L), w.rope_base)
        kv[b] = (k, f64(inp.v[b], dt))

    def fn(row):
        b, i = row
        lo = max(0, i - W + 1)
        q = f64(inp.q[b, i], dt)[None]  # [1, Hq, dqk]
        if w.rope_base:
            q = oracle.apply_rope(q, [i], w.rope_base)
        qs = np.zeros((1, i - lo + 1) + q.shape[1:])
        qs[0, -1] = q[0]  # the row sits at the end of its key slice; earlier rows are not read
        k, v = kv[b]
        ro, rl = oracle.prefill_rows(qs, k[None, lo:i + 1], v[None, lo:i + 1], W, inp.sink, inp.scale,
                                     [(0, i - lo)])
        return ErrorSums().add(o_host[b, i].double().numpy()[None], ro, lse_host[b, :, i].numpy()[None], rl)

    return run_units(fn, rows)


def decode_all(w, inp, o_host, lse_host):
    """Every output of a decode: a unit is one (sequence, KV head) - its G query heads, its cache
    column and new tokens, as a one-KV-head problem for the oracle. o_host [B, T, Hq, dv], lse_host
    [B, T, Hq]."""
    dt = w.dtype
    G = w.Hq // w.Hkv

    def fn(unit):
        b, g = unit
        heads = np.arange(g * G, (g + 1) * G)
        sel = lambda x, idx: f64(x[b:b + 1][:, :, idx], dt)
        args = (sel(inp.q, heads), sel(inp.k_new, [g]), sel(inp.v_new, [g]), sel(inp.k_cache, [g]),
                sel(inp.v_cache, [g]), inp.cache_len[b:b + 1],
                None if inp.cache_offset is None else inp.cache_offset[b:b + 1], w.window,
                inp.sink[heads], inp.scale)
        if w.rope_base:
            ro, rl = oracle.decode_rope(*args, w.rope_base)
        else:
            ro, rl = oracle.decode(*args)
        got = o_host[b:b + 1, :, g * G:(g + 1) * G].double().numpy()
        got_lse = lse_host[b:b + 1, :, g * G:(g + 1) * G].numpy()
        return ErrorSums().add(got, ro, got_lse, rl)

    return run_units(fn, [(b, g) for b in range(w.B) for g in range(w.Hkv)])
