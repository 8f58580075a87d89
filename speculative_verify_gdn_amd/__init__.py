"""MI355X-native (gfx950) speculative-verify step of one Gated-DeltaNet layer.

The compute path is the HIP library ``libgdn.so`` (C ABI declared in
``include/gdn.h``); ``speculative_verify_gdn_amd.gdn`` is a thin ctypes
binding over it that marshals torch device tensors and the current stream.
Importing this package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""
__all__ = ["gdn", "synth"]
