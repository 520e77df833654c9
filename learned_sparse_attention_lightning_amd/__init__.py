"""DeepSeek Sparse Attention forward path for AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libdsa.so``); this package only loads it and marshals torch tensors into
its calls.  Importing the package does not touch the GPU.
"""
__all__ = ["configs", "synth"]
