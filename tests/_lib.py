"""Loads the built library for tests, building it first if it is missing."""

import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "zero_partition_aware_amd", "libzr.so")


def load():
    if not os.path.exists(LIB):
        from zero_partition_aware_amd import build
        build.build()
    from zero_partition_aware_amd import zr
    return zr
