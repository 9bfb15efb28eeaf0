"""rotated_w8a8_int8_amd -- rotated W8A8 int8 linear layer for AMD MI355X (gfx950).

The compute lives in ``librad.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/rad.h``).  ``binding`` is a thin ctypes layer over it
that passes device pointers and the caller's stream; ``workloads`` draws the
seeded synthetic inputs.  Importing the package loads nothing: the library is
opened on the first call into ``binding`` and that call raises if it is not
built.
"""
__all__ = ["binding", "workloads"]
