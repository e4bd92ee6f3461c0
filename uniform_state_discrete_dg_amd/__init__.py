"""libdgdenoise: uniform-state text-diffusion denoising on MI355X (gfx950).

The compute path is the C-ABI library ``libdgdenoise.so`` (hand-written HIP
kernels, declared in ``include/dgdenoise.h``).  ``binding`` is a thin ctypes
layer with the same entry-point names; PyTorch only supplies device memory
and streams.  ``workloads`` holds the seeded synthetic inputs.  Nothing here
loads the shared library until an entry point is first called.
"""
__all__ = ["binding", "workloads"]
