"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only draws random numbers and rounds them to the storage dtype. It holds none of the
attention arithmetic: neither the kernels nor the oracle import anything from each other, and both
receive exactly the arrays produced here.

Recipe (stated once, used everywhere):

* Every tensor is a stream of float32 ``standard_normal`` draws. The stream for tensor ``name`` of
  seed ``seed`` is split into fixed chunks of 2**22 elements; chunk ``c`` is drawn from
  ``Generator(PCG64(SeedSequence([seed, STREAM_IDS[name]]).spawn(n_chunks)[c]))``. The chunking makes
  parallel generation deterministic: the values never depend on the number of threads.
* bf16 tensors are the float32 draws rounded to nearest-even bfloat16. They are kept as raw 16-bit
  patterns (``uint16``); ``bf16_to_f32`` widens them exactly.
* Decode lengths and ring offsets are integers drawn from their own streams.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22

STREAM_IDS = {
    "sink": 0,
    "q": 1,
    "k": 2,
    "v": 3,
    "k_new": 4,
    "v_new": 5,
    "k_cache": 6,
    "v_cache": 7,
    "cache_len": 8,
    "cache_offset": 9,
    "d_o": 10,
}


def host_threads() -> int:
    """Threads for input generation: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, returning the 16-bit patterns (finite inputs)."""
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array holding the nearest-even bfloat16 values."""
    return bf16_to_f32(_f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)))


def normal(seed: int, name: str, shape, dtype: str = "f32", threads: int | None = None) -> np.ndarray:
    """Seeded N(0,1) tensor. dtype 'f32' -> float32 array; 'bf16' -> uint16 bit patterns."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    if n == 0:
        return out.reshape(shape)
    n_chunks = (n + CHUNK - 1) // CHUNK
    children = np.random.SeedSequence([int(seed), STREAM_IDS[name]]).spawn(n_chunks)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(children[c]))
        if dtype == "bf16":
            tmp = g.standard_normal(hi - lo, dtype=np.float32)
            out[lo:hi] = _f32_to_bf16_bits(tmp)
        else:
            g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    nt = threads or host_threads()
    if n_chunks == 1 or nt == 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(min(nt, n_chunks)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def integers(seed: int, name: str, shape, low: int, high: int) -> np.ndarray:
    """Seeded int32 tensor, uniform on [low, high)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), STREAM_IDS[name]])))
    return g.integers(low, high, size=shape, dtype=np.int64).astype(np.int32)


def as_float(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of an input array: bf16 bit patterns are widened, float32 is returned as is."""
    return bf16_to_f32(arr) if dtype == "bf16" else arr


@dataclass
class PrefillInputs:
    dtype: str
    q: np.ndarray  # [B, L, Hq, dqk]  (uint16 bf16 bits or float32)
    k: np.ndarray  # [B, L, Hkv, dqk]
    v: np.ndarray  # [B, L, Hkv, dv]
    sink: np.ndarray | None  # [Hq] float32
    scale: float
    window: int


@dataclass
class DecodeInputs:
    dtype: str
    q: np.ndarray  # [B, T, Hq, dqk]
    k_new: np.ndarray  # [B, T, Hkv, dqk]
    v_new: np.ndarray  # [B, T, Hkv, dv]
    k_cache: np.ndarray  # [B, C, Hkv, dqk]
    v_cache: np.ndarray  # [B, C, Hkv, dv]
    cache_len: np.ndarray  # [B] int32
    cache_offset: np.ndarray | None  # [B] int32
    sink: np.ndarray | None  # [Hq] float32
    scale: float
    window: int
    extra: dict = field(default_factory=dict)


def prefill_inputs(seed, B, L, Hq, Hkv, dqk, dv, window, dtype="bf16", with_sink=True,
                   scale=None, threads=None) -> PrefillInputs:
    """Draw order: sink, q, k, v (each from its own stream, so the order only documents intent)."""
    sink = normal(seed, "sink", (Hq,), "f32") if with_sink else None
    q = normal(seed, "q", (B, L, Hq, dqk), dtype, threads)
    k = normal(seed, "k", (B, L, Hkv, dqk), dtype, threads)
    v = normal(seed, "v", (B, L, Hkv, dv), dtype, threads)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    return PrefillInputs(dtype, q, k, v, sink, float(scale), int(window))


def output_grad(seed, B, L, Hq, dv, dtype="bf16", threads=None) -> np.ndarray:
    """Seeded upstream gradient dO [B, L, Hq, dv] of the prefill output (N(0,1), own stream)."""
    return normal(seed, "d_o", (B, L, Hq, dv), dtype, threads)


def decode_inputs(seed, B, T, Hq, Hkv, dqk, dv, C, window, dtype="bf16", cache_len=None,
                  len_range=None, ring_offsets=True, with_sink=True, scale=None,
                  threads=None) -> DecodeInputs:
    """Draw order: sink, q, k_new, v_new, k_cache, v_cache, cache_len, cache_offset.

    ``cache_len`` fixes every sequence's committed length; otherwise lengths are uniform on
    ``len_range = (low, high)``. With ``ring_offsets`` each sequence gets a uniform offset in [0, C).
    """
    sink = normal(seed, "sink", (Hq,), "f32") if with_sink else None
    q = normal(seed, "q", (B, T, Hq, dqk), dtype, threads)
    k_new = normal(seed, "k_new", (B, T, Hkv, dqk), dtype, threads)
    v_new = normal(seed, "v_new", (B, T, Hkv, dv), dtype, threads)
    k_cache = normal(seed, "k_cache", (B, C, Hkv, dqk), dtype, threads)
    v_cache = normal(seed, "v_cache", (B, C, Hkv, dv), dtype, threads)
    if cache_len is not None:
        lens = np.full((B,), int(cache_len), dtype=np.int32)
    else:
        lo, hi = len_range
        lens = integers(seed, "cache_len", (B,), lo, hi)
    offs = integers(seed, "cache_offset", (B,), 0, C) if ring_offsets else None
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    return DecodeInputs(dtype, q, k_new, v_new, k_cache, v_cache, lens, offs, sink, float(scale),
                        int(window))


def to_torch(arr: np.ndarray, dtype: str, device="cuda"):
    """Upload an input array as a torch tensor of the storage dtype (bf16 from bit patterns)."""
    import torch

    if arr is None:
        return None
    if dtype == "bf16" and arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)
