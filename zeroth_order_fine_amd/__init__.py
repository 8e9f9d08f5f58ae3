"""MI355X-native inference-native zeroth-order candidate scoring.

The product is libzo.so (HIP kernels for gfx950 behind the C-ABI in
include/zo.h); this package is its thin Python binding.  Importing works
without the library; any call that needs it raises if libzo.so is missing.
"""
from . import api
from .api import (Bank, DeviceBatch, Model, Plan, ZoError, bank_cap, batch_layout, direction, estimate, fold, generate,
                  normal_fill,
                  pack, philox_words, score, update)

__all__ = ["api", "Bank", "DeviceBatch", "Model", "Plan", "ZoError", "batch_layout", "direction", "estimate",
           "fold", "generate", "normal_fill", "pack", "philox_words", "score", "update"]
