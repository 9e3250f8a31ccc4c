"""MI355X-native Reformer LSH-attention forward pass.

The four steps (hash, sort, chunked attention, unsort + round combine) are
HIP kernels for gfx950 behind the C ABI declared in ``include/lsh.h``
(library ``liblsh.so`` in this package).  ``binding`` is the thin Python
marshalling layer over that ABI; ``synth`` draws the seeded synthetic inputs.
Importing the package loads nothing; the library is opened on first use.
"""
__all__ = ["binding", "synth"]
