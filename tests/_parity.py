"""Shared helpers for GPU-vs-oracle parity tests (inputs from the seeded generator only)."""

from __future__ import annotations

import sys

import numpy as np

from sliding_window_sink_seeded_amd.inputs import as_float, to_torch

# Tolerances stated for the method: fp32 inputs -> relative error 1e-5 (max-norm and L2);
# bf16 inputs with fp32 accumulation -> max |err| <= 2e-2 and relative L2 <= 5e-3.
TOL = {
    "f32": dict(rel_max=1e-5, rel_l2=1e-5, lse_abs=2e-5),
    "bf16": dict(abs_max=2e-2, rel_l2=5e-3, lse_abs=2e-3),
}

# Gradients of the backward pass, at the same bars. Gradient magnitudes are not O(1) (dk sums over
# every query of a window and every head of a group), so the bf16 max-error bar is taken relative
# to the largest reference entry: max |err| <= 2e-2 max |ref|, relative L2 <= 5e-3. fp32: relative
# max-norm and L2 errors <= 1e-5. Sink gradient: a sum of B * L terms exp(s_h - lse_i) D_i whose
# sum can cancel, so its error is taken relative to the mass sum_i exp(s_h - lse_i) sum_d |dO o|;
# bf16 rounds o before D is formed (relative 2^-9 per element) -> 4e-3, fp32 -> 1e-5.
GRAD_TOL = {"f32": dict(rel_max=1e-5, rel_l2=1e-5), "bf16": dict(rel_max=2e-2, rel_l2=5e-3)}
SINK_TOL = {"f32": 1e-5, "bf16": 4e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    ref_max = float(np.abs(ref).max()) if ref.size else 0.0
    ref_l2 = float(np.linalg.norm(ref))
    return dict(
        abs_max=float(np.abs(d).max()) if d.size else 0.0,
        rel_max=(float(np.abs(d).max()) / ref_max) if ref_max > 0 else float(np.abs(d).max()),
        rel_l2=(float(np.linalg.norm(d)) / ref_l2) if ref_l2 > 0 else float(np.linalg.norm(d)),
        finite=bool(np.isfinite(got).all()),
    )


def assert_output_close(got, ref, dtype, what="o"):
    m = metrics(got, ref)
    tol = TOL[dtype]
    assert m["finite"], f"{what}: non-finite values"
    if dtype == "f32":
        ok = m["rel_max"] <= tol["rel_max"] and m["rel_l2"] <= tol["rel_l2"]
    else:
        ok = m["abs_max"] <= tol["abs_max"] and m["rel_l2"] <= tol["rel_l2"]
    assert ok, f"{what}: {m} exceeds {tol}"
    return m


def assert_grad_close(got, ref, dtype, what):
    m = metrics(got, ref)
    tol = GRAD_TOL[dtype]
    assert m["finite"], f"{what}: non-finite values"
    assert m["rel_max"] <= tol["rel_max"] and m["rel_l2"] <= tol["rel_l2"], f"{what}: {m} vs {tol}"
    return m


def sink_grad_rel_err(dsink, ref_dsink, d_o, ref_o, ref_lse, sink):
    """Per-head sink-gradient error relative to the mass of the terms it sums (see SINK_TOL)."""
    Dabs = np.einsum("bihd,bihd->bhi", np.abs(d_o), np.abs(ref_o))
    mass = (np.exp(np.asarray(sink, np.float64)[None, :, None] - ref_lse) * Dabs).sum(axis=(0, 2))
    return np.abs(np.asarray(dsink, np.float64) - ref_dsink) / np.maximum(mass, 1e-30)


def assert_lse_close(got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    assert np.isfinite(got).all() and err <= TOL[dtype]["lse_abs"], f"lse err {err}"
    return err


def torch_dtype(dtype):
    import torch

    return torch.bfloat16 if dtype == "bf16" else torch.float32


def gpu_from_numpy(arr, dtype):
    return to_torch(arr, dtype, "cuda")


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def f(arr, dtype):
    """Exact float values of a generator array."""
    return as_float(arr, dtype)
