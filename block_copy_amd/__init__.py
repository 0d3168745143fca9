"""block_copy_amd -- batched descriptor copy for AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``libkvcopy.so`` (header: include/kvcopy.h),
built from ``csrc/`` by ``block_copy_amd.build``.  ``block_copy_amd.kvcopy``
is its ctypes binding; importing it loads the library and fails loudly if it
is missing.  This package file itself loads nothing.
"""
