"""MI355X (gfx950) decoder for entropy-coded Int8 / FP8 weight streams.

The compute path is libeq.so (hand-written HIP for CDNA4, C ABI in
include/eq.h); ``rans_decode_amd.eq`` is its Python binding. Importing the
binding loads the library and raises if it is missing; there is no CPU
fallback.
"""
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libeq.so")

__all__ = ["LIB_PATH"]
