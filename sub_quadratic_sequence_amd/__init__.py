"""MI355X-native chunkwise Gated Linear Attention (forward, backward, decode step)
and the chunkwise Gated DeltaNet forward.

The compute lives in hand-written HIP kernels for gfx950 behind the C ABI of
``libgla.so`` (declared in ``include/gla.h``).  ``gla`` is the thin ctypes
binding over it; ``inputs`` draws seeded synthetic workloads.  Importing the
package loads nothing: the library is opened on the first call.
"""

__all__ = ["gla_chunk_fwd", "gla_recurrent_step", "gla_chunk_bwd", "gdn_chunk_fwd"]


def __getattr__(name):
    if name in __all__:
        from . import gla

        return getattr(gla, name)
    raise AttributeError(name)
