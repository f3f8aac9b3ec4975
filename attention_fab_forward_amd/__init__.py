"""MI355X-native fused two-matmul block O = f(A.B).C (attention and GeLU MLP).

The compute lives in libfab.so (hand-written HIP for gfx950 behind a C ABI,
declared in include/fab.h); this package holds the build script, a thin ctypes
binding and the seeded synthetic-input generator.
"""
from ._binding import (FabError, Plan, backward, forward, lib, make_problem, merge,  # noqa: F401
                       ulysses_pack, ulysses_sequence_view, ulysses_sizes, ulysses_unpack)

__all__ = ["forward", "backward", "merge", "ulysses_pack", "ulysses_unpack", "ulysses_sizes",
           "ulysses_sequence_view", "Plan", "FabError", "lib", "make_problem"]
