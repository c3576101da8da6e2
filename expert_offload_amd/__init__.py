"""MI355X-native routed-expert MoE layer with an expert cache.

The compute path is libmoe.so (HIP for gfx950, C ABI in include/moe.h);
this package holds its ctypes binding (same entry-point names), the build
script, and a small helper that assembles a whole layer from the entry
points.  Nothing here computes on the CPU.
"""
from . import _lib
from ._lib import *  # noqa: F401,F403
from ._lib import (Cache, Ctx, MoeError, QTYPE, EXPORTS, lib, make_ffn_args,  # noqa: F401
                   moe_ffn_args)

__all__ = [n for n in dir(_lib) if not n.startswith("_")]
