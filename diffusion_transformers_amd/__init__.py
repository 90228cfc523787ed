"""BinaryAttention forward pass, native on AMD MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/binattn.h``).  ``binding`` is a thin ctypes
layer over it that uses PyTorch only for device memory and streams; import it
explicitly (``from diffusion_transformers_amd import binding``) -- importing the
package itself loads nothing.
"""
__all__ = ["binding", "workloads"]
