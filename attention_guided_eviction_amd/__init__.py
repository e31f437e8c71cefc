"""Beacon-guided KV-cache compression on AMD Instinct MI355X (gfx950).

The compute lives in libbkv.so (hand-written HIP kernels behind the C ABI of
include/bkv.h); `bkv` is its ctypes binding and `event` runs one whole compression
event over a model's layers.
"""
from . import bkv  # noqa: F401
from .event import CompressionEvent  # noqa: F401

__all__ = ["bkv", "CompressionEvent"]
