"""fp64 CPU oracle for DiffQKV attention -- test infrastructure only.

Imported by the test-suite, the smoke check and the benchmark's CPU-baseline
leg; never by the GPU library.
"""

from .attention import (attend_one, attend_selective_one, attention_weights, decode,
                        decode_paged, decode_selective, default_scale, group_sharing_index,
                        kv_append, kv_group_sharing, paged_to_contiguous, prefill,
                        prefill_all_rows, top_k_rows)

from .augq import augq, silu

__all__ = ["augq", "silu", "attend_one", "attend_selective_one", "attention_weights", "decode",
           "decode_paged", "decode_selective", "default_scale", "group_sharing_index",
           "kv_append", "kv_group_sharing", "paged_to_contiguous", "prefill",
           "prefill_all_rows", "top_k_rows"]
