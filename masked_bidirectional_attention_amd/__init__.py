"""Masked bidirectional attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libmzattn.so`` (hand-written HIP, C ABI declared in
``include/mzattn.h``); this package only marshals torch tensors into it.

    from masked_bidirectional_attention_amd import mzattn_fwd, mzattn_decode, mzattn_decode_append
"""
from ._binding import (  # noqa: F401
    DecodeAppendCall,
    DecodeCall,
    FwdCall,
    LIB_PATH,
    MzattnError,
    MzattnNotBuilt,
    lib,
    mzattn_decode,
    mzattn_decode_append,
    mzattn_decode_noalloc,
    mzattn_device_info,
    mzattn_fwd,
)

__all__ = ["DecodeCall", "DecodeAppendCall", "FwdCall", "mzattn_fwd", "mzattn_decode", "mzattn_decode_append", "mzattn_decode_noalloc", "mzattn_device_info", "MzattnError", "MzattnNotBuilt", "lib", "LIB_PATH"]
