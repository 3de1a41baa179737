"""CPU oracle of the DSA indexer decode step -- test infrastructure only.

Importable by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``; never by the product path. Shares no code with the HIP
library.
"""
from .indexer import (PAGE, bf16_bits_to_f64, clamp_len, e4m3_to_f64, gather_keys, key_histogram, order_keys, score,
                      score_at, score_fp8, score_magnitudes, score_magnitudes_fp8, score_magnitudes_mtp,
                      score_mtp, sparse_attention, topk, topk_values)

__all__ = ["PAGE", "bf16_bits_to_f64", "clamp_len", "e4m3_to_f64", "gather_keys", "key_histogram", "order_keys", "score",
           "score_at", "score_fp8", "score_magnitudes", "score_magnitudes_fp8", "score_magnitudes_mtp",
           "score_mtp", "sparse_attention", "topk", "topk_values"]
