"""MI355X (gfx950) TriAttention KV-cache eviction pass.

Score -> GQA aggregate -> select -> in-place compaction, behind the C ABI of
include/tria.h (libtria.so, hand-written HIP kernels).  ``tria`` is the
ctypes binding; ``synth`` makes seeded synthetic caches and statistics.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "tria", "build"]
