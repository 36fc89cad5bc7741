"""MI355X-native Speculative Pipeline Decoding: the single-GPU hot path.

The compute path is libspd.so (HIP kernels for gfx950 behind the C ABI in
include/spd.h); this package only marshals arguments to it.
"""
from .binding import (SPD, SpdError, balance_stages, load, make_config, upload_weights, LIB_PATH,
                      SYMBOLS, OP_NAMES, DBG)

__all__ = ["SPD", "SpdError", "balance_stages", "load", "make_config", "upload_weights",
           "LIB_PATH", "SYMBOLS", "OP_NAMES", "DBG"]
