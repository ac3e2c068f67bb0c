"""MI355X-native Parallel Transformer Block (PTB) layer: forward and backward.

The compute lives in ``libptb.so`` (hand-written HIP kernels for gfx950 behind a
C ABI declared in ``include/ptb.h``).  ``transformer_block_amd.ptb`` is the thin
ctypes binding over it; importing this package does not load the library.
"""
__all__ = ["inputs", "flops"]
