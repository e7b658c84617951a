"""Mixed-precision AdamW optimizer step for AMD MI355X (gfx950).

libhpo.so (C ABI in include/hpo.h, HIP kernels in csrc/) does all the work;
`hpo` is its ctypes binding and `optimizer` orders one step the way the pages
do.  `inputs` draws the seeded synthetic workloads.
"""
from . import hpo  # noqa: F401
from .optimizer import DeviceAdamW, MixedPrecisionAdamW  # noqa: F401

__all__ = ["hpo", "MixedPrecisionAdamW", "DeviceAdamW"]
