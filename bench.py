#!/usr/bin/env python3
"""Benchmark of the sink-seeded SWA / global attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the attention over one batch of seeded synthetic input already resident in
HBM. The headline workload is the sliding-window bf16 prefill (batch 4 x 32768, 64/8 heads, W=128):
`value` is algorithmic TFLOP/s (only visible scores, 640 FLOP each) over the wall clock of the K
timed steps. One JSON line goes to stdout, with:

* roofline - the dominant kernel's algorithmic bytes (or FLOPs) per launch divided by its average
  launch duration, timed with HIP events on the launch stream, against MI355X's published peak;
* cpu_baseline - the float64 oracle timed on the host cores (a pool of forked worker processes,
  one per core up to 16) over a bounded leading sample of the same workload, for the headline and
  every other workload (a reported baseline, not a target);
* secondary - the other measured workloads (fp32 prefill, global prefill, ring decode, split-KV
  global decode, both decodes at the 16K-context / 64-sequence MTP setting, the four bf16
  workloads with the rotary embedding fused, both decodes with 8-token block drafts, the commit
  of 8 accepted tokens into the sliding-window rings, and the backward pass of both bf16
  prefills),
  timed the same way, with decode inputs rotated over enough copies to defeat the 256 MiB MALL.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA peaks, TFLOP/s
MALL_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = os.path.join(ROOT, "sliding_window_sink_seeded_amd", "csrc")

METRIC = "prefill attn TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"

# the other measured workloads, in the order they are timed
SECONDARY = ("swa_prefill_f32", "ga_prefill_bf16", "swa_decode_bf16", "ga_decode_bf16",
             "swa_decode_mtp_bf16", "ga_decode_mtp_bf16", "swa_prefill_rope_bf16",
             "ga_prefill_rope_bf16", "swa_decode_rope_bf16", "ga_decode_rope_bf16",
             "swa_decode_t8_bf16", "ga_decode_t8_bf16", "swa_backward_bf16", "ga_backward_bf16")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Case:
    """Seeded inputs for one workload, uploaded once (plus rotated copies), and its launcher."""

    def __init__(self, w, rotate_to_defeat_mall=True):
        import numpy as np
        import torch

        import sliding_window_sink_seeded_amd as mimo
        from sliding_window_sink_seeded_amd import inputs, workloads

        self.w = w
        self.mimo = mimo
        dt = w.dtype
        t0 = time.perf_counter()
        if w.kind in ("prefill", "backward"):
            self.inp = inputs.prefill_inputs(w.seed, w.B, w.L, w.Hq, w.Hkv, w.dqk, w.dv, w.window, dt)
            self.d_o = inputs.output_grad(w.seed, w.B, w.L, w.Hq, w.dv, dt) if w.kind == "backward" else None
            self.lens = None
            self.flops, self.bytes = workloads.algorithmic(w)
        else:
            self.inp = inputs.decode_inputs(w.seed, w.B, w.T, w.Hq, w.Hkv, w.dqk, w.dv, w.C, w.window,
                                            dt, cache_len=(w.P or None),
                                            len_range=(w.len_range or None),
                                            ring_offsets=w.ring_offsets)
            self.lens = self.inp.cache_len
            self.flops, self.bytes = workloads.algorithmic(w, self.lens)
        log(f"[bench] {w.name}: inputs generated in {time.perf_counter() - t0:.1f} s")
        up = lambda x: inputs.to_torch(x, dt)
        n_sets = 1
        if rotate_to_defeat_mall and self.bytes < 4 * MALL_BYTES:
            n_sets = min(16, max(2, math.ceil(8 * MALL_BYTES / self.bytes)))
        self.sink = torch.from_numpy(self.inp.sink).cuda()
        self.rope = None
        if w.rope_base > 0:  # built once, outside the timed region, like a model's cos/sin cache
            n_pos = w.L if w.kind == "prefill" else int(w.P or w.len_range[1]) + w.T
            self.rope = mimo.rope_table(n_pos, w.rope_base)
        self.sets = []
        if w.kind == "backward":
            # the forward's o and lse are inputs of the backward: computed once, untimed
            base = [up(self.inp.q), up(self.inp.k), up(self.inp.v)]
            self.d_o_t = up(self.d_o)
            o, lse = mimo.prefill(base[0], base[1], base[2], w.window, sink=self.sink,
                                  scale=self.inp.scale, return_lse=True)
            self.fwd = (o, lse)
            self.ws = torch.empty(mimo.backward_workspace_size(w.B, w.L, w.Hq), dtype=torch.uint8,
                                  device="cuda")
            for i in range(n_sets):
                ts = base if i == 0 else [t.clone() for t in base]
                self.sets.append((ts, tuple(torch.empty_like(t) for t in ts)))
        elif w.kind == "prefill":
            base = [up(self.inp.q), up(self.inp.k), up(self.inp.v)]
            for i in range(n_sets):
                ts = base if i == 0 else [t.clone() for t in base]
                o = torch.empty(w.B, w.L, w.Hq, w.dv, dtype=ts[0].dtype, device="cuda")
                self.sets.append((ts, o))
        else:
            base = [up(self.inp.q), up(self.inp.k_new), up(self.inp.v_new), up(self.inp.k_cache),
                    up(self.inp.v_cache)]
            self.len_t = torch.from_numpy(self.inp.cache_len).cuda()
            self.off_t = (torch.from_numpy(self.inp.cache_offset).cuda()
                          if self.inp.cache_offset is not None else None)
            self.max_len = int(w.P or w.len_range[1])
            nb = mimo.decode_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.dv, self.max_len, w.window)
            self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
            for i in range(n_sets):
                ts = base if i == 0 else [t.clone() for t in base]
                o = torch.empty(w.B, w.T, w.Hq, w.dv, dtype=ts[0].dtype, device="cuda")
                self.sets.append((ts, o))
        self.n_sets = n_sets
        self.i = 0
        torch.cuda.synchronize()

    def run(self):
        ts, o = self.sets[self.i % self.n_sets]
        self.i += 1
        w = self.w
        if w.kind == "backward":
            return self.mimo.prefill_backward(ts[0], ts[1], ts[2], self.fwd[0], self.fwd[1], self.d_o_t,
                                              w.window, sink=self.sink, scale=self.inp.scale,
                                              workspace=self.ws, out=o)
        if w.kind == "prefill":
            self.mimo.prefill(ts[0], ts[1], ts[2], w.window, sink=self.sink, scale=self.inp.scale, out=o,
                              rope=self.rope)
        else:
            self.mimo.decode(ts[0], ts[1], ts[2], ts[3], ts[4], self.len_t, w.window, self.max_len,
                             cache_offset=self.off_t, sink=self.sink, scale=self.inp.scale,
                             workspace=self.ws, out=o, rope=self.rope)
        return o

    def time(self, steps, warmup, min_warm_s=0.25):
        """W untimed warm-up steps (continued until min_warm_s has passed, so clocks have
        settled), then exactly `steps` timed steps. Returns the mean wall-clock and HIP-event time
        per step; the per-step event times (an event between consecutive steps, on the launch
        stream) are kept in self.step_ms for their median and minimum."""
        import torch

        t0 = time.perf_counter()
        n = 0
        while n < warmup or time.perf_counter() - t0 < min_warm_s:
            self.run()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        evs[0].record()
        for k in range(steps):
            self.run()
            evs[k + 1].record()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        event_ms = evs[0].elapsed_time(evs[-1]) / steps
        self.step_ms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(steps))
        return wall_ms, event_ms

    def time_back_to_back(self, steps):
        """GPU time per step with the host out of the way: `steps` steps are queued behind device
        copies (256 MB each, keeping the GPU and its memory busy) that outlast their enqueueing,
        so the GPU runs them back to back; the events bracket the steps only. Short kernels
        launched one call at a time from Python otherwise leave launch gaps inside the per-step
        event times. Returns None when the copies could not be made to outlast the enqueueing."""
        import torch

        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        n_copies = 8
        try:
            for _ in range(3):
                torch.cuda.synchronize()
                ev_busy, ev0, ev1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                ev_busy.record()
                for _ in range(n_copies):
                    dst.copy_(src)
                ev0.record()
                t0 = time.perf_counter()
                for _ in range(steps):
                    self.run()
                ev1.record()
                host_ms = (time.perf_counter() - t0) * 1e3
                torch.cuda.synchronize()
                if ev_busy.elapsed_time(ev0) > 1.25 * host_ms:
                    return ev0.elapsed_time(ev1) / steps
                n_copies *= 4
            return None
        finally:
            del src, dst

    def sampled_parity(self, n_rows=8):
        """Compare a few output rows (all heads) with the oracle; returns error metrics."""
        import numpy as np
        import torch

        import oracle
        from sliding_window_sink_seeded_amd.inputs import as_float

        w, inp, dt = self.w, self.inp, self.w.dtype
        self.i = 0  # every rotated set holds the same inputs; use the first
        o = self.run()
        torch.cuda.synchronize()
        if w.kind == "backward":
            # dq of a few rows (all heads); the oracle reads only the sequences they lie in
            dq = o[0]
            rows = [(0, 0), (0, min(w.L - 1, 128)), (w.B - 1, w.L // 2), (w.B - 1, w.L - 1)]
            got, ref = [], []
            for b, i in rows:
                args = [as_float(x[b:b + 1], dt) for x in (inp.q, inp.k, inp.v, self.d_o)]
                ref.append(oracle.backward_rows(*args, w.window, inp.sink, inp.scale, [(0, i)])[0])
                got.append(dq[b, i].float().cpu().numpy())
            got, ref = np.stack(got), np.stack(ref)
        elif w.kind == "prefill":
            rng = np.random.default_rng(0)
            pos = sorted({0, w.L - 1, min(w.L - 1, 127), min(w.L - 1, 128),
                          *rng.integers(0, w.L, n_rows - 4).tolist()})
            rows = [(int(b), int(i)) for b, i in zip(rng.integers(0, w.B, len(pos)), pos)]
            got = np.stack([o[b, i].float().cpu().numpy() for b, i in rows])
            ref = []
            for b, i in rows:
                # row i sees keys [lo, i]: it is the last row of that slice of the sequence
                lo = max(0, i - w.window + 1)
                rq = _pad_q(as_float(inp.q[b:b + 1, i:i + 1], dt), i - lo)
                rk = as_float(inp.k[b:b + 1, lo:i + 1], dt)
                rv = as_float(inp.v[b:b + 1, lo:i + 1], dt)
                ro, _ = oracle.prefill_rows(rq, rk, rv, w.window, inp.sink, inp.scale, [(0, i - lo)])
                ref.append(ro[0])
            ref = np.stack(ref)
        else:
            seqs = [0, w.B - 1]
            keep = list(range(0, w.Hq, 7))
            got = o[seqs].float().cpu().numpy()[:, :, keep]
            ref, _ = oracle.decode(as_float(inp.q[seqs], dt), as_float(inp.k_new[seqs], dt),
                                   as_float(inp.v_new[seqs], dt), as_float(inp.k_cache[seqs], dt),
                                   as_float(inp.v_cache[seqs], dt), inp.cache_len[seqs],
                                   None if inp.cache_offset is None else inp.cache_offset[seqs],
                                   w.window, inp.sink, inp.scale, heads=keep)
            ref = ref[:, :, keep]
        d = got.astype(np.float64) - ref
        return {"rows": int(np.prod(got.shape[:-1])), "abs_max": float(np.abs(d).max()),
                "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref))}


def time_cache_append(steps=50):
    """Commit of 8 accepted tokens per sequence into the 128-slot rings of the sliding-window
    decode workload (256 sequences, 8 KV heads): HIP-event time per call and the bytes it moves
    (each K/V row read once from the new-token tensors and written once into the ring)."""
    import torch

    import sliding_window_sink_seeded_amd as mimo
    from sliding_window_sink_seeded_amd import inputs, workloads

    w = workloads.WORKLOADS["swa_decode_t8_bf16"]
    inp = inputs.decode_inputs(w.seed, w.B, w.T, w.Hq, w.Hkv, w.dqk, w.dv, w.C, w.window, w.dtype,
                               len_range=w.len_range, ring_offsets=True)
    up = lambda x: inputs.to_torch(x, w.dtype)
    kn, vn, kc, vc = up(inp.k_new), up(inp.v_new), up(inp.k_cache), up(inp.v_cache)
    lens = torch.from_numpy(inp.cache_len).cuda()
    offs = torch.from_numpy(inp.cache_offset).cuda()
    for _ in range(5):  # the rings keep wrapping: every call is a full commit
        mimo.cache_append(kn, vn, kc, vc, lens, (1 << 30) - 8, cache_offset=offs)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        mimo.cache_append(kn, vn, kc, vc, lens, (1 << 30) - 8, cache_offset=offs)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    nbytes = 2 * w.B * w.T * w.Hkv * (w.dqk + w.dv) * w.elem
    return {"workload": "swa_cache_append_t8_bf16", "kernel_ms": round(ms, 4),
            "algorithmic_bytes": nbytes, "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "description": "commit of 8 accepted tokens x 256 sequences x 8 KV heads into 128-slot rings"}


def _pad_q(rq, n_before):
    """Place one query row at slice position n_before (earlier rows are never read)."""
    import numpy as np

    q = np.zeros((1, n_before + 1) + rq.shape[2:], dtype=rq.dtype)
    q[:, n_before] = rq[:, 0]
    return q


# ------------------------------------------------------------------ CPU baseline: the oracle

# The workload, its inputs and the deadline of the CPU baseline being timed. Set before the worker
# processes are forked (before anything touches the GPU), so the workers inherit it.
_JOB = {}


def cpu_workers():
    """(worker processes, cores visible): the cores this process may run on, at most 16 workers
    (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n)), n


def _one_blas_thread():
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)


def _cpu_unit(unit):
    """One unit of oracle work in a worker; returns (algorithmic FLOPs, algorithmic bytes) done,
    (0, 0) when the unit starts past the deadline."""
    import numpy as np

    import oracle
    from sliding_window_sink_seeded_amd import workloads
    from sliding_window_sink_seeded_amd.inputs import as_float

    if time.perf_counter() > _JOB["deadline"]:
        return 0, 0
    w, inp = _JOB["w"], _JOB["inp"]
    f64 = lambda x: np.asarray(as_float(x, w.dtype), np.float64)
    G = w.Hq // w.Hkv
    if unit[0] == "rows":  # prefill rows [i0, i1) of sequence b, query heads of KV head g
        _, b, i0, i1, g = unit
        lo = max(0, i0 - w.window + 1)
        q = f64(inp.q[b, i0:i1, g * G:(g + 1) * G])
        k, v = f64(inp.k[b, lo:i1, g]), f64(inp.v[b, lo:i1, g])
        if w.rope_base:
            q = oracle.apply_rope(q, np.arange(i0, i1), w.rope_base)
            k = oracle.apply_rope(k, np.arange(lo, i1), w.rope_base)
        for j in range(G):
            oracle.sink_attention(q[:, j], np.arange(i0, i1), k, np.arange(lo, i1), v,
                                  float(inp.sink[g * G + j]), inp.scale, w.window)
        scores = sum(min(i + 1, w.window) for i in range(i0, i1)) * G
        return scores * 2 * (w.dqk + w.dv), 0
    if unit[0] == "head":  # backward of one query head over the leading S rows of sequence 0
        _, h, S = unit
        g = h // G
        sl = lambda x, j: f64(x[0:1, :S, j:j + 1])
        oracle.prefill_backward(sl(inp.q, h), sl(inp.k, g), sl(inp.v, g), sl(_JOB["d_o"], h),
                                w.window, inp.sink[h:h + 1], inp.scale)
        return workloads.prefill_scores(1, S, 1, w.window) * 2 * (3 * w.dqk + 2 * w.dv), 0
    _, b, g = unit  # decode: sequence b, KV head g with its G query heads
    heads = np.arange(g * G, (g + 1) * G)
    sel = lambda x, idx: f64(x[b:b + 1][:, :, idx])
    args = (sel(inp.q, heads), sel(inp.k_new, [g]), sel(inp.v_new, [g]), sel(inp.k_cache, [g]),
            sel(inp.v_cache, [g]), inp.cache_len[b:b + 1],
            None if inp.cache_offset is None else inp.cache_offset[b:b + 1], w.window,
            inp.sink[heads], inp.scale)
    if w.rope_base:
        oracle.decode_rope(*args, w.rope_base)
    else:
        oracle.decode(*args)
    P = int(inp.cache_len[b])
    flops = workloads.decode_scores(inp.cache_len[b:b + 1], w.T, G, w.window) * 2 * (w.dqk + w.dv)
    nbytes = (w.T * G * (w.dqk + w.dv) + (min(P, w.window - 1) + w.T) * (w.dqk + w.dv)) * w.elem
    return flops, nbytes


def cpu_baseline(w, target_s):
    """The float64 oracle as it stands, timed on the host over a bounded leading sample of workload
    `w`, on a pool of forked worker processes (one BLAS thread each). Must run before the GPU is
    initialised: the workers are forked from this process.

    Units are dealt in order; those that would start after `target_s` are skipped, so the sample is
    a leading part of the workload (prefill: rows of sequence 0 onwards; decode: (sequence, KV
    head) pairs from sequence 0 on). The backward pass runs every query head over the leading S rows
    of sequence 0, S sized by a one-head probe. The rate is in the workload's own unit: TFLOP/s of
    visible scores for prefills and backward passes, GB/s of algorithmic bytes for decodes."""
    import multiprocessing as mp

    from sliding_window_sink_seeded_amd import inputs

    workers, visible = cpu_workers()
    dt = w.dtype
    if w.kind in ("prefill", "backward"):
        inp = inputs.prefill_inputs(w.seed, w.B, w.L, w.Hq, w.Hkv, w.dqk, w.dv, w.window, dt)
        d_o = inputs.output_grad(w.seed, w.B, w.L, w.Hq, w.dv, dt) if w.kind == "backward" else None
    else:
        inp = inputs.decode_inputs(w.seed, w.B, w.T, w.Hq, w.Hkv, w.dqk, w.dv, w.C, w.window, dt,
                                   cache_len=(w.P or None), len_range=(w.len_range or None),
                                   ring_offsets=w.ring_offsets)
        d_o = None
    _JOB.clear()
    _JOB.update(w=w, inp=inp, d_o=d_o, deadline=float("inf"))
    if w.kind == "backward":
        # one head over 256 rows in this process, then S so that all heads take about target_s
        t0 = time.perf_counter()
        _cpu_unit(("head", 0, 256))
        t1 = max(time.perf_counter() - t0, 1e-3)
        per_head = target_s * workers / w.Hq
        grow = per_head / t1 if w.window < w.L else math.sqrt(per_head / t1)
        S = int(min(w.L, max(256, (256 * grow) // 256 * 256)))
        units = [("head", h, S) for h in range(w.Hq)]
        sample = f"sequence 0, rows [0, {S}) of {w.L}, every one of {w.Hq} heads"
    elif w.kind == "prefill":
        units = [("rows", b, i0, min(w.L, i0 + 256), g) for b in range(w.B) for i0 in range(0, w.L, 256)
                 for g in range(w.Hkv)]
    else:
        units = [("kv", b, g) for b in range(w.B) for g in range(w.Hkv)]
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_one_blas_thread) as pool:
        pool.map(_noop, range(workers))  # worker start-up, untimed
        # the workers hold copies of _JOB made at the fork: the deadline travels with each unit
        deadline = time.perf_counter() + target_s if w.kind != "backward" else float("inf")
        t0 = time.perf_counter()
        done = pool.map(_cpu_timed_unit, [(u, deadline) for u in units], chunksize=1)
        secs = time.perf_counter() - t0
    flops = sum(f for f, _ in done)
    nbytes = sum(b for _, b in done)
    n_done = sum(1 for f, _ in done if f > 0)
    if w.kind == "prefill":
        sample = (f"the first {n_done} (block of 256 rows, KV head) units, sequence-major, of "
                  f"{w.B} x {w.L} rows x {w.Hkv} KV heads (about {n_done * 256 // w.Hkv} rows, "
                  f"all {w.Hq} query heads)")
    elif w.kind == "decode":
        sample = f"the first {n_done} of {w.B} x {w.Hkv} (sequence, KV head) pairs, all {w.T} tokens"
    used = min(workers, len(units))
    if w.kind == "decode":
        value, unit = nbytes / secs / 1e9, "GB/s"
    else:
        value, unit = flops / secs / 1e12, "TFLOP/s"
    _JOB.clear()
    return {"value": value, "unit": unit, "cores": used, "kind": "oracle", "sample": sample,
            "seconds": round(secs, 2), "workers": "processes (fork), 1 BLAS thread each",
            "host_cores_visible": visible}


def _noop(_):
    return None


def _cpu_timed_unit(arg):
    unit, deadline = arg
    _JOB["deadline"] = deadline
    return _cpu_unit(unit)


def kernel_source_digest(kind):
    """sha256 over the HIP sources (names and bytes) that build and launch the `kind` kernels."""
    import hashlib

    own = {"prefill": ["tiles.hpp", "prefill.hip"], "backward": ["tiles.hpp", "backward.hip"]}
    names = ["api.hip", "common.hpp", "launch.hpp"] + own.get(kind, ["decode.hip"])
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, kind):
    """HBM bytes per launch of the workload's dominant kernel from its committed counter summary
    (FETCH_SIZE / WRITE_SIZE, scaled by a plain copy's counters), or None when there is no summary
    or the kernel sources have changed since the counters were taken."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_digest(kind):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def describe(case, wall_ms, event_ms, b2b_ms=None):
    w = case.w
    tflops = case.flops / (wall_ms * 1e-3) / 1e12
    gbs = case.bytes / (event_ms * 1e-3) / 1e9
    steps = getattr(case, "step_ms", None) or [event_ms]
    d = {
        "workload": w.name, "ms_per_step": round(wall_ms, 4), "kernel_ms": round(event_ms, 4),
        "kernel_ms_median": round(statistics.median(steps), 4), "kernel_ms_min": round(steps[0], 4),
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS[w.dtype], 4),
        "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_flop": case.flops, "algorithmic_bytes": case.bytes,
        "rotated_input_sets": case.n_sets,
    }
    if b2b_ms:
        # the same steps run back to back on the GPU (no host launch gaps)
        d["kernel_ms_back_to_back"] = round(b2b_ms, 4)
        d["hbm_frac_back_to_back"] = round(case.bytes / (b2b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        d["mfma_frac_back_to_back"] = round(case.flops / (b2b_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 4)
    return d


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="swa_prefill_bf16")
    ap.add_argument("--no-secondary", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="wall-clock bound of the headline workload's CPU baseline")
    ap.add_argument("--cpu-seconds-secondary", type=float, default=1.0,
                    help="wall-clock bound of each other workload's CPU baseline")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--warm-seconds", type=float, default=0.25,
                    help="keep warming up (untimed) until this much time has passed")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sharding is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from sliding_window_sink_seeded_amd import workloads

    names = [args.workload] + ([] if args.no_secondary else [n for n in SECONDARY if n != args.workload])
    cpu = {}
    if not args.no_cpu_baseline:
        # first, before anything touches the GPU: the oracle's worker processes fork from here
        for name in names:
            t0 = time.perf_counter()
            cpu[name] = cpu_baseline(workloads.WORKLOADS[name],
                                     args.cpu_seconds if name == args.workload else args.cpu_seconds_secondary)
            log(f"[bench] {name}: cpu baseline {cpu[name]} ({time.perf_counter() - t0:.1f} s with inputs)")

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = workloads.WORKLOADS[args.workload]

    if args.calibrate_copy:
        # a plain copy kernel of known size: reads 1 GiB and writes 1 GiB per launch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    case = Case(w)
    wall_ms, event_ms = case.time(args.steps, args.warmup, args.warm_seconds)
    head = describe(case, wall_ms, event_ms)
    log(f"[bench] {w.name}: {head}")
    parity = None if args.no_parity else case.sampled_parity()

    if w.kind in ("prefill", "backward") and w.window < w.L:
        bound, unit = "hbm", "GB/s"
        achieved, peak, per_launch = case.bytes / (event_ms * 1e-3) / 1e9, HBM_PEAK_GBS, case.bytes
    elif w.kind in ("prefill", "backward"):
        bound, unit = "mfma", "TFLOP/s"
        achieved, peak, per_launch = case.flops / (event_ms * 1e-3) / 1e12, MFMA_PEAK_TFLOPS[w.dtype], case.flops
    else:
        bound, unit = "hbm", "GB/s"
        achieved, peak, per_launch = case.bytes / (event_ms * 1e-3) / 1e9, HBM_PEAK_GBS, case.bytes
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name, w.kind),
                "algorithmic_per_launch": per_launch, "kernel_avg_ms": round(event_ms, 4)}

    del case
    torch.cuda.empty_cache()

    secondary = []
    if not args.no_secondary:
        for name in names[1:]:
            c = Case(workloads.WORKLOADS[name])
            sw, se = c.time(max(5, args.steps // 2), 3, args.warm_seconds)
            b2b = c.time_back_to_back(max(5, args.steps // 2))
            d = describe(c, sw, se, b2b)
            d["cpu_baseline"] = cpu.get(name)
            log(f"[bench] {name}: {d}")
            secondary.append(d)
            del c
            torch.cuda.empty_cache()

    if not args.no_secondary:
        d = time_cache_append()
        log(f"[bench] cache append: {d}")
        secondary.append(d)

    tflops = head["algorithmic_flop"] / (wall_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs rounded to bf16; sink N(0,1) fp32)",
        "config": {"workload": w.description, "name": w.name, "batch": w.B, "seq_len": w.L or None,
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "d_qk": w.dqk, "d_v": w.dv,
                   "window": w.window, "parallelism": "single GPU"},
        "mfma_frac": head["mfma_frac"],
        "hbm_frac": head["hbm_frac"],
        "kernel_ms_median": head["kernel_ms_median"],
        "kernel_ms_min": head["kernel_ms_min"],
        "roofline": roofline,
        "cpu_baseline": cpu.get(w.name),
        "parity": parity,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
