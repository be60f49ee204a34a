"""MI355X-native fused Linear -> Swish -> +bias -> GroupNorm.

The compute lives in a HIP shared library (``liblgn.so``, C ABI declared in
``include/lgn.h``); ``gemm_activation_groupnorm_amd.lgn`` is the thin ctypes
binding with the same entry-point names.  Importing this package loads nothing.
"""
