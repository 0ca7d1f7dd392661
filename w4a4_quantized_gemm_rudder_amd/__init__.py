"""Stream-aware W4A8/W4A4 linear layer for AMD Instinct MI355X (gfx950).

The compute lives in librudder.so (HIP kernels behind the C ABI of
include/rudder.h); `rudder` is its Python binding and `workloads` draws the
seeded synthetic inputs.  Submodules are imported on demand so that loading
the input generator never requires the HIP library.
"""
__all__ = ["rudder", "workloads", "build"]
