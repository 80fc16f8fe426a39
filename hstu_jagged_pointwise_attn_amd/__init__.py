"""HSTU jagged pointwise attention on MI355X (gfx950).

The compute path is the C-ABI library ``libhstu.so`` (hand-written HIP
kernels); ``api`` marshals torch tensors into it. Importing this package does
not load the library; the first call does, and fails loudly if it is missing.
"""
