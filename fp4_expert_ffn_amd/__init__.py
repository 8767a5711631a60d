"""Routed FP4 expert FFN for AMD MI355X (gfx950).

The computation lives in the HIP library ``libmoe_fp4.so`` behind the C ABI of
``include/moe_fp4.h``; :mod:`fp4_expert_ffn_amd.moe_fp4` is its ctypes binding and
:mod:`fp4_expert_ffn_amd.device` the device-memory plumbing around it.
"""

from . import moe_fp4  # noqa: F401  (loads the library lazily, on first call)

__all__ = ["moe_fp4"]
