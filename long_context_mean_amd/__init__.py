"""MISA routed indexer on MI355X (gfx950).

The compute path is the HIP library libmisa.so (C ABI declared in
include/misa.h); `long_context_mean_amd.binding` passes torch device tensors
and the current HIP stream to it, and `synth` draws seeded inputs.  Importing
the package does not load the library; the first op call does, and raises if
the library is missing.
"""
from . import synth  # noqa: F401
