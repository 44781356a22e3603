"""Float64 CPU oracle for KV-cache maintenance around decode / MTP verification.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (same rules as ``oracle.attention``): only the test suite,
the smoke check and the bench's CPU-baseline leg may import it; it shares no code with the HIP
library.

What the pages fix
------------------
* MiMo series notes (plmsmile), MiMo-V2-Flash > lightweight MTP > inference: drafted tokens are
  verified by the main model in one pass; only the accepted ones continue the sequence.
* Same notes, MiMo-V2.6 / DFlash ablations: block drafts of 6 or 8 tokens are verified at once.
* jienda explainer, §4.3 (memory management): the sliding-window layers keep a fixed-size KV
  cache; the global layers keep the whole history.

Readings taken where the pages are silent (listed again in the design notes):
* The cache holds committed tokens only; position p of sequence b lives in slot (p + off_b) mod C
  (the decode oracle's convention). A verify step reads its T new tokens from separate tensors.
* Committing: after the verify step, the first a_b of the T new tokens (the accepted prefix,
  0 <= a_b <= T) are written at positions P_b .. P_b + a_b - 1 and the committed length becomes
  P_b + a_b. Rejected drafts are rolled back by never being written: the cache afterwards is the
  cache of the accepted sequence.
* A linear cache is the ring with off_b = 0 and no position reaching C.
"""

from __future__ import annotations

import numpy as np


def cache_append(k_new, v_new, k_cache, v_cache, cache_len, cache_offset=None, accept=None):
    """Commit the accepted prefix of the T new tokens of every sequence.

    k_new [B, T, Hkv, dqk], v_new [B, T, Hkv, dv]; k_cache [B, C, Hkv, dqk], v_cache
    [B, C, Hkv, dv]; cache_len [B]; cache_offset [B] or None (0); accept [B] or None (all T).
    Returns (k_cache', v_cache', cache_len') as new arrays; the inputs are not modified.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    lens = np.array(cache_len, dtype=np.int64, copy=True)
    B, T = np.shape(k_new)[:2]
    C = kc.shape[1]
    for b in range(B):
        a = T if accept is None else int(accept[b])
        if not 0 <= a <= T:
            raise ValueError("accepted count outside [0, T]")
        off = 0 if cache_offset is None else int(cache_offset[b])
        for t in range(a):
            slot = (int(lens[b]) + t + off) % C
            kc[b, slot] = k_new[b, t]
            vc[b, slot] = v_new[b, t]
        lens[b] += a
    return kc, vc, lens
