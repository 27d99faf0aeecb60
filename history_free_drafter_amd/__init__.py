"""DLite draft step on AMD Instinct MI355X (gfx950).

The compute lives in libdlite.so (HIP kernels behind the C ABI of
include/dlite.h); `binding` marshals arguments to it and `runtime` holds the
device-side buffers (torch tensors used as plain device memory).
"""
__all__ = ["binding", "runtime"]
