"""HiLS (Hierarchical Landmark Sparse) attention forward pass for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libhils.so`` (hand-written HIP kernels); ``hils`` is its
thin Python binding and ``synth`` draws seeded synthetic inputs.  Importing the package loads
nothing: the library is opened on first use of ``hils`` and its absence is an error.
"""
__all__ = ["hils", "synth"]
