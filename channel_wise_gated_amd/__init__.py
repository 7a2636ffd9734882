"""channel_wise_gated_amd -- the channel-wise gated delta rule on MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI of
``libgdr.so`` (declared in ``include/gdr.h``); ``channel_wise_gated_amd.gdr``
is the thin ctypes binding with the same entry-point names.  Importing this
package does not load the library; the binding loads it on first use and
raises if it is missing.
"""
__all__ = ["gdr", "inputs"]
