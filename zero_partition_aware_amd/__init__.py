"""Partition-aware ZeRO-1/2 gradient reduction for MI355X (gfx950).

The compute path is the C-ABI library ``libzr.so`` (HIP kernels plus a host
planner); ``zero_partition_aware_amd.zr`` is its thin ctypes binding and
``zero_partition_aware_amd.workloads`` holds the seeded synthetic inputs.
Importing the package loads nothing; importing ``.zr`` loads the library and
raises if it has not been built.
"""

__all__ = ["zr", "workloads"]
