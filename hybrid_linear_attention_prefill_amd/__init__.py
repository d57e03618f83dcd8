"""MI355X-native chunked Gated DeltaNet prefill with grid-exact, forkable state.

The compute runs in ``libgdn_prefill.so`` (hand-written HIP for gfx950 behind a C ABI,
declared in ``include/gdn.h``).  :mod:`.binding` is a thin ctypes layer over that library;
:mod:`.synth` makes seeded synthetic inputs.  Importing this package loads nothing native;
``from hybrid_linear_attention_prefill_amd import binding`` does, and raises if the library
has not been built.
"""
__all__ = ["binding", "synth"]
