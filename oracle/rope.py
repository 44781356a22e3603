"""Float64 CPU oracle for the partial rotary position embedding applied to Q and K.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (same rules as ``oracle.attention``): only the test suite,
the smoke check and the bench's CPU-baseline leg may import it; it shares no code with the HIP
library.

What the pages fix
------------------
* MiMo-V2-Flash Technical Report review (xllm-io), §3.1: RoPE is applied to the first 64 of the
  192 query/key dimensions only.
* Same page, §4 (pre-training, hyper-parameters): RoPE base 10K for the sliding-window layers;
  640K raised to 5M for the global layers by the last stage.
* MiMo series notes (plmsmile), MiMo-V2-Flash paper summary > pre-training and context extension >
  window extension: the global layers' RoPE setting is changed for 256K, the local layers keep
  their small window.

Readings taken where the pages are silent (listed again in the design notes):
* Rotation layout: the rotated 64 dimensions form 32 pairs (i, i + 32), i = 0..31 ("rotate half"
  within the rotated slice); dimensions 64..191 pass through unchanged.
* Frequencies: inv_freq_i = base^(-2i / 64); angle = position * inv_freq_i.
* Positions: the absolute token position within its sequence (prefill row i -> i; decode token t
  of a sequence with P committed tokens -> P + t). V is never rotated.
* The cache holds keys already rotated (they were rotated when their token was processed), so a
  decode step rotates only its own Q and new K.

For a pair (x, y) at position p and frequency index i, with a = p * inv_freq_i:
    x' = x cos a - y sin a,     y' = y cos a + x sin a
"""

from __future__ import annotations

import numpy as np

ROT_DIMS = 64  # rotated leading dimensions of each Q/K head vector


def inv_freq(base: float, rot_dims: int = ROT_DIMS) -> np.ndarray:
    """inv_freq_i = base^(-2i / rot_dims) for i = 0 .. rot_dims/2 - 1, in float64."""
    i = np.arange(rot_dims // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / rot_dims)


def angles(positions, base: float, rot_dims: int = ROT_DIMS) -> np.ndarray:
    """[n, rot_dims/2] rotation angles position * inv_freq_i (float64)."""
    p = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    return p * inv_freq(base, rot_dims)[None, :]


def rope_table(n_pos: int, base: float, rot_dims: int = ROT_DIMS) -> np.ndarray:
    """[n_pos, rot_dims/2, 2] (cos, sin) of the angles of positions 0 .. n_pos-1 (float64)."""
    a = angles(np.arange(n_pos), base, rot_dims)
    return np.stack([np.cos(a), np.sin(a)], axis=-1)


def apply_rope(x, positions, base: float, rot_dims: int = ROT_DIMS) -> np.ndarray:
    """Rotate the leading rot_dims of the last axis of x.

    x: [n, d] or [n, H, d] with n tokens at the given positions ([n]). Returns a float64 copy.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if x.ndim not in (2, 3):
        raise ValueError("x must be [n, d] or [n, H, d]")
    half = rot_dims // 2
    a = angles(positions, base, rot_dims)  # [n, half]
    if x.ndim == 3:
        a = a[:, None, :]  # same angle for every head of a token
    c, s = np.cos(a), np.sin(a)
    lo = x[..., :half].copy()
    hi = x[..., half:rot_dims].copy()
    x[..., :half] = lo * c - hi * s
    x[..., half:rot_dims] = hi * c + lo * s
    return x


def prefill_rope(q, k, v, window, sink, scale, base, kv_head_of_q=None, return_real=False):
    """Prefill of pre-rotation Q/K: rotate Q and K by their row positions, then attend.

    q [B, L, Hq, dqk], k [B, L, Hkv, dqk], v [B, L, Hkv, dv].
    """
    from .attention import prefill

    L = np.shape(q)[1]
    pos = np.arange(L)
    qr = np.stack([apply_rope(qb, pos, base) for qb in np.asarray(q, dtype=np.float64)])
    kr = np.stack([apply_rope(kb, pos, base) for kb in np.asarray(k, dtype=np.float64)])
    return prefill(qr, kr, v, window, sink, scale, kv_head_of_q=kv_head_of_q, return_real=return_real)


def decode_rope(q, k_new, v_new, k_cache, v_cache, cache_len, cache_offset, window, sink, scale,
                base, kv_head_of_q=None, seqs=None, heads=None):
    """Decode with pre-rotation Q and new K (positions P_b + t); the cache holds rotated keys."""
    from .attention import decode

    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    T = q.shape[1]
    qr = np.empty_like(q)
    kr = np.empty_like(k_new)
    for b in range(q.shape[0]):
        pos = int(cache_len[b]) + np.arange(T)
        qr[b] = apply_rope(q[b], pos, base)
        kr[b] = apply_rope(k_new[b], pos, base)
    return decode(qr, kr, v_new, k_cache, v_cache, cache_len, cache_offset, window, sink, scale,
                  kv_head_of_q=kv_head_of_q, seqs=seqs, heads=heads)
