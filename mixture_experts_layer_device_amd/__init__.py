"""One-GPU MoE layer hot path for AMD MI355X (gfx950).

The compute lives in ``libmk.so`` (hand-written HIP kernels behind the C ABI
of ``include/mk.h``); ``binding`` marshals arguments to it (importing it
raises if the library is not built -- there is no fallback) and ``layer``
holds the device-memory plumbing (torch tensors as buffers, streams).
``build`` compiles the library and does not load it.
"""
__all__ = ["binding", "layer", "build"]
