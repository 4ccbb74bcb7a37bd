"""MI355X (gfx950) flow-matching action-expert denoise loop.

The compute path is the HIP library ``libvla_expert.so`` (C ABI in
``include/vla_expert.h``); this package only builds it and marshals
arguments to it.  Importing ``binding`` or ``expert`` requires the built
library and raises if it is missing: there is no CPU fallback.
"""
__all__ = ["binding", "expert", "build"]
