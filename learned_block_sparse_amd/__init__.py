"""MiniMax Sparse Attention (MSA) on MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libmsa.so``, declared in ``include/msa.h``); ``learned_block_sparse_amd.msa``
is its thin Python binding.  Importing this package does not load the library;
the first call through the binding does, and fails loudly if it is missing.
"""
__all__ = ["msa", "synth"]
