"""fp64 CPU oracle for R-SWA (test infrastructure only; see rswa.py's header)."""
from .rswa import (FULL, RSWA, attend, brute_decode, brute_prefill, cache_ratio, decode_step,
                   decode_visible, default_scale, full_cache_rows, full_row, paged_prefix, prefill,
                   prefill_backward, prefill_lse, prefill_visible, queue_decode, ring_occupants,
                   ring_row, rswa_cache_rows, softmax_grad)

__all__ = ["FULL", "RSWA", "attend", "brute_decode", "brute_prefill", "cache_ratio",
           "decode_step", "decode_visible", "default_scale", "full_cache_rows", "full_row",
           "paged_prefix",
           "prefill", "prefill_backward", "prefill_lse", "prefill_visible", "queue_decode",
           "ring_occupants", "ring_row", "rswa_cache_rows", "softmax_grad"]
