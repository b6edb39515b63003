"""Batch-1 Dual-AR (RQ-Transformer) decode frame on MI355X (gfx950).

The compute path is the HIP library `libdar.so` built from `csrc/` and reached
through its C ABI (`include/dar.h`). `native` holds the ctypes binding with the
same names as the C entry points; importing it loads the library and raises if
it is missing. This top-level module imports nothing native so that host-only
helpers (`bytes_model`) stay importable without a build.
"""
__all__ = ["bytes_model"]
