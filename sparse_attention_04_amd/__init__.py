"""MI355X-native DSA hot path: fused Lightning Indexer + Top-K + Sparse Flash
Attention behind a C ABI (``include/dsa.h``).  The HIP library is loaded lazily
by :mod:`sparse_attention_04_amd.binding`; importing this package loads nothing.
"""
__all__ = ["binding", "inputs"]
