"""MI355X-native fused add + argmax readout (``xpress_add_argmax_to_blk``).

The computation runs in hand-written HIP kernels for gfx950 behind a C-ABI
shared library (``libxpress_argmax.so``, declared in ``include/xpress_argmax.h``).
``vocab_wide_add_amd.native`` is the thin ctypes binding with the same entry
point names; it raises if the library has not been built -- there is no
fallback path.
"""
__version__ = "0.1.0"
