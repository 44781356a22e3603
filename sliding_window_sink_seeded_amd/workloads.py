"""The measured workloads and their algorithmic work.

Shapes follow the MiMo-V2-Flash Technical Report review (xllm-io), §3.1: window 128; 64 query heads
over 8 KV heads for sliding-window layers and over 4 KV heads for global layers; Q/K head dim 192,
V head dim 128. Decode carries 1 + 3 draft tokens per sequence (same page, §2: three MTP layers used
as the self-speculative draft), and the global decode runs at the 256K context of the same page §1.

Algorithmic work counts only what the method must do:
* FLOPs: 2 * (dqk + dv) per visible (query, key) score; nothing masked or skipped is counted.
  The backward pass counts five products per visible score, 2 * (3 dqk + 2 dv): the scores
  q.k (recomputed, as every attention backward that does not store P does), dO.v, and the
  contributions to dV, dK and dQ.
* Bytes: Q read once, the union of visible K/V read once, new K/V read once, O written once.
  Backward: Q, K, V, O, dO and lse read once, dQ, dK, dV written once.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill", "decode" or "backward" (of a prefill)
    dtype: str  # "f32" or "bf16"
    Hq: int
    Hkv: int
    window: int
    dqk: int = 192
    dv: int = 128
    B: int = 1
    L: int = 0  # prefill sequence length
    T: int = 0  # decode: new tokens per sequence
    C: int = 0  # decode: cache slots per sequence
    P: int = 0  # decode: fixed committed length (0 -> drawn from len_range)
    len_range: tuple = ()  # decode: committed lengths uniform on [lo, hi)
    ring_offsets: bool = False
    seed: int = 0
    description: str = ""
    rope_base: float = 0.0  # > 0: Q/K given before the rotary embedding (first 64 dims, this base)

    @property
    def elem(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dqk)


WORKLOADS = {
    "swa_prefill_f32": Workload(
        "swa_prefill_f32", "prefill", "f32", 64, 8, 128, B=1, L=512, seed=1,
        description="sliding-window prefill fp32, batch 1 x 512, 64/8 heads, W=128"),
    "swa_prefill_bf16": Workload(
        "swa_prefill_bf16", "prefill", "bf16", 64, 8, 128, B=4, L=32768, seed=2,
        description="sliding-window prefill bf16, batch 4 x 32768, 64/8 heads, W=128"),
    "ga_prefill_bf16": Workload(
        "ga_prefill_bf16", "prefill", "bf16", 64, 4, 32768, B=1, L=32768, seed=3,
        description="global causal prefill bf16, batch 1 x 32768, 64/4 heads"),
    "swa_decode_bf16": Workload(
        "swa_decode_bf16", "decode", "bf16", 64, 8, 128, B=256, T=4, C=128,
        len_range=(128, 32768), ring_offsets=True, seed=4,
        description="sliding-window decode bf16, 256 seqs x 4 tokens, 128-slot ring, 64/8 heads"),
    "ga_decode_bf16": Workload(
        "ga_decode_bf16", "decode", "bf16", 64, 4, 1 << 30, B=8, T=4, C=262144, P=262144, seed=5,
        description="global decode bf16, 8 seqs x 262144 cached + 4 tokens, 64/4 heads, split-KV"),
    # The pages' own MTP measurement setting: 16K-token inputs, 64 sequences per node, 1 + 3
    # drafts verified per step (MiMo-V2-Flash Technical Report review (xllm-io), §6.3; MiMo series
    # notes (plmsmile), MiMo-V2-Flash paper summary > evaluation and system experiments, and > MTP
    # decode gains).
    "swa_decode_mtp_bf16": Workload(
        "swa_decode_mtp_bf16", "decode", "bf16", 64, 8, 128, B=64, T=4, C=128, P=16384,
        ring_offsets=True, seed=6,
        description="sliding-window decode bf16, 64 seqs x 16384 cached + 4 tokens, 128-slot ring, 64/8 heads"),
    "ga_decode_mtp_bf16": Workload(
        "ga_decode_mtp_bf16", "decode", "bf16", 64, 4, 1 << 30, B=64, T=4, C=16384, P=16384, seed=7,
        description="global decode bf16, 64 seqs x 16384 cached + 4 tokens, 64/4 heads, split-KV"),
}

# Block-draft verification (MiMo series notes (plmsmile), MiMo-V2.6 decoding ablation: DFlash
# blocks of 6 and 8 tokens): the two bf16 decode workloads with 8 new tokens per sequence.
for _name in ("swa_decode_bf16", "ga_decode_bf16"):
    _w = WORKLOADS[_name]
    _tn = _name.replace("_bf16", "_t8_bf16")
    WORKLOADS[_tn] = Workload(**{**_w.__dict__, "name": _tn, "T": 8,
                                 "description": _w.description.replace("x 4 tokens", "x 8 tokens")
                                 .replace("+ 4 tokens", "+ 8 tokens") + " (block draft of 8)"})

# The training backward pass of the two bf16 prefill workloads (MiMo-V2-Flash Technical Report
# review (xllm-io), §3.2: the sink logit is learned, so its gradient is computed too).
WORKLOADS["swa_backward_bf16"] = Workload(
    "swa_backward_bf16", "backward", "bf16", 64, 8, 128, B=4, L=32768, seed=2,
    description="sliding-window backward bf16 (dq, dk, dv, dsink), batch 4 x 32768, 64/8 heads, W=128")
WORKLOADS["ga_backward_bf16"] = Workload(
    "ga_backward_bf16", "backward", "bf16", 64, 4, 32768, B=1, L=32768, seed=3,
    description="global causal backward bf16 (dq, dk, dv, dsink), batch 1 x 32768, 64/4 heads")

# The same four bf16 workloads with Q/K given before the rotary embedding, rotated inside the
# kernels (MiMo-V2-Flash Technical Report review (xllm-io), §3.1 and §4: first 64 dims, base 10K for
# sliding-window layers, 5M for global layers). Same inputs (same seeds) as the plain workloads.
for _name, _base in (("swa_prefill_bf16", 1e4), ("ga_prefill_bf16", 5e6), ("swa_decode_bf16", 1e4),
                     ("ga_decode_bf16", 5e6)):
    _w = WORKLOADS[_name]
    _rn = _name.replace("_bf16", "_rope_bf16")
    WORKLOADS[_rn] = Workload(**{**_w.__dict__, "name": _rn, "rope_base": _base,
                                 "description": _w.description + f", RoPE base {_base:g} fused"})


def prefill_scores(B: int, L: int, Hq: int, window: int) -> int:
    """Visible (query, key) pairs of a prefill: row i sees min(i + 1, W) keys."""
    w = min(window, L)
    per_head = w * (w + 1) // 2 + (L - w) * w
    return B * Hq * per_head


def prefill_bytes(w: Workload) -> int:
    e = w.elem
    q = w.B * w.L * w.Hq * w.dqk * e
    kv = w.B * w.L * w.Hkv * (w.dqk + w.dv) * e
    o = w.B * w.L * w.Hq * w.dv * e
    return q + kv + o


def decode_scores(lens: np.ndarray, T: int, Hq: int, window: int) -> int:
    total = 0
    for P in np.asarray(lens, dtype=np.int64):
        for t in range(T):
            total += min(int(P) + t + 1, window)
    return int(total * Hq)


def decode_bytes(w: Workload, lens: np.ndarray) -> int:
    e = w.elem
    committed = sum(min(int(P), w.window - 1) for P in np.asarray(lens, dtype=np.int64))
    q = w.B * w.T * w.Hq * w.dqk * e
    cache = committed * w.Hkv * (w.dqk + w.dv) * e
    new = w.B * w.T * w.Hkv * (w.dqk + w.dv) * e
    o = w.B * w.T * w.Hq * w.dv * e
    return q + cache + new + o


def backward_bytes(w: Workload) -> int:
    e = w.elem
    per_row = w.Hq * (w.dqk + 2 * w.dv) * e + w.Hq * 4  # reads: q, o, dO, lse
    per_row += w.Hkv * (w.dqk + w.dv) * e                # reads: k, v
    per_row += w.Hq * w.dqk * e + w.Hkv * (w.dqk + w.dv) * e  # writes: dq, dk, dv
    return w.B * w.L * per_row


def algorithmic(w: Workload, lens: np.ndarray | None = None) -> tuple[int, int]:
    """(FLOPs, bytes) of one pass over workload ``w`` (decode needs the drawn lengths)."""
    per_score = 2 * (w.dqk + w.dv)
    if w.kind == "backward":
        return (prefill_scores(w.B, w.L, w.Hq, w.window) * 2 * (3 * w.dqk + 2 * w.dv),
                backward_bytes(w))
    if w.kind == "prefill":
        return prefill_scores(w.B, w.L, w.Hq, w.window) * per_score, prefill_bytes(w)
    return decode_scores(lens, w.T, w.Hq, w.window) * per_score, decode_bytes(w, lens)
