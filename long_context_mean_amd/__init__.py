"""MISA routed indexer on MI355X (gfx950).

The compute path is the HIP library libmisa.so (C ABI declared in
include/misa.h).  `binding` passes torch device tensors and the current HIP
stream to it; `synth` draws seeded inputs.  Importing this package does not
load the library; the first call of an op does, and raises if it is missing.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "binding"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    raise AttributeError(name)
