"""Affine 3/4-bit group-64 quantized matmul y = x . W^T for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libqmm.so`` (hand-written HIP kernels);
``binding`` is a thin ctypes layer over it that uses PyTorch only for device
memory and streams. Importing this package does not load the library; the
first call into ``binding`` does, and fails loudly if it is missing.
"""
__all__ = ["synth", "binding"]


def __getattr__(name):
    if name in ("binding", "synth"):
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
