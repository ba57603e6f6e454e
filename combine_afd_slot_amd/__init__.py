"""MI355X-native FFN-rank hot path of Attention-FFN Disaggregation (AFD).

The compute path lives in the HIP library ``libafd.so`` (built from
``csrc/``) behind the C ABI declared in ``include/afd.h``; ``afd`` is its thin
ctypes binding.  Importing this package loads nothing: the library is opened on
first use of ``combine_afd_slot_amd.afd``, and fails loudly when it is missing.
"""

__all__ = ["afd", "inputs"]
