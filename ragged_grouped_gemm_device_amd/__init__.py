"""MI355X-native dropless MoE expert MLP on a sync-free ragged grouped GEMM.

The compiled library (``libmoe.so``, C ABI declared in ``include/moe.h``) does
all of the work; ``ragged_grouped_gemm_device_amd.moe`` is a thin ctypes
binding over it. Importing this package loads nothing.
"""
