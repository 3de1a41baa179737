"""MI355X-native DSA indexer decode step.

``binding`` is the thin ctypes layer over ``libdsa_indexer.so`` (the C-ABI
declared in ``include/dsa_indexer.h``); ``workloads`` draws the seeded
synthetic inputs. Importing the package loads nothing native; the library is
loaded on first use of ``binding`` and a missing library is an error.
"""
__all__ = ["binding", "workloads"]
