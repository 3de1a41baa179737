"""CPU oracle of the DSA indexer decode step -- test infrastructure only.

Importable by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``; never by the product path. Shares no code with the HIP
library.
"""
from .indexer import (PAGE, bf16_bits_to_f64, clamp_len, gather_keys, score,
                      score_at, score_magnitudes, topk, topk_values)

__all__ = ["PAGE", "bf16_bits_to_f64", "clamp_len", "gather_keys", "score",
           "score_at", "score_magnitudes", "topk", "topk_values"]
