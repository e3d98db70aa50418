"""Invariant Bit Packing (IBP) for AMD Instinct MI355X.

The C ABI lives in include/ibp.h and libibp.so (HIP kernels for gfx950);
`lossless_bit_level_amd.ibp` is its ctypes binding.
"""
