"""Float64 CPU oracle (test infrastructure only; see ``oracle.attention``)."""

from .attention import (combine, decode, decode_keys, default_kv_map, prefill, prefill_rows,
                        sink_attention, split_partials, visible)
from .backward import backward_keys, backward_rows, prefill_backward
from .cache import cache_append
from .rope import ROT_DIMS, apply_rope, decode_rope, inv_freq, prefill_rope, rope_table

__all__ = ["combine", "decode", "decode_keys", "default_kv_map", "prefill", "prefill_rows",
           "sink_attention", "split_partials", "visible", "backward_keys", "backward_rows",
           "prefill_backward", "cache_append", "ROT_DIMS", "apply_rope", "decode_rope", "inv_freq", "prefill_rope",
           "rope_table"]
