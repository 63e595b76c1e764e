"""STILL intra-layer hybrid attention, forward path, for MI355X (gfx950).

The compute path lives in the C-ABI library ``libstill.so`` (hand-written HIP
kernels); :mod:`linear_attention_still_amd.still` is its thin ctypes binding.
Importing the package loads nothing: the library is opened on first use.
"""
__all__ = ["inputs", "still"]
