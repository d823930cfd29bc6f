"""MI355X-native sparse decode over tiered KV (SPIN-style decode step).

The compute path lives in the HIP library ``libspin.so`` (C-ABI declared in
``include/spin.h``); ``binding`` is its thin ctypes wrapper and ``workload``
draws seeded synthetic inputs.  Importing the package loads nothing; import
``sparse_attention_tiered_amd.binding`` to load the library.
"""
__all__ = ["binding", "workload"]
