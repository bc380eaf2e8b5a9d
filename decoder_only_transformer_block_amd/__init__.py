"""MI355X-native (gfx950) pre-norm decoder block: forward and backward in
hand-written HIP kernels behind the C ABI of libdtb.so (include/dtb.h).

Submodules: `binding` (ctypes marshalling of the C ABI), `runtime` (torch
buffers for a block stack), `configs` / `inputs` (the seeded synthetic
workloads), `build` (hipcc build of libdtb.so)."""
__all__ = ["binding", "configs", "inputs", "build", "runtime"]
