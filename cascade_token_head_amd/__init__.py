"""MI355X (gfx950) cascade token/head pruned attention.

libspatten.so (built from csrc/ by `python -m cascade_token_head_amd.build`)
holds every kernel behind a C ABI (include/spatten.h); `spatten` is the
ctypes binding and `pipeline` sequences the calls over a layer stack.
"""
from . import spatten  # noqa: F401
