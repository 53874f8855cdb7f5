"""MI355X-native chunked-prefill mixed step: host batch builder + gfx950 kernels behind libcb.so.

``binding`` mirrors the C ABI of ``include/cb.h`` (and ``include/cb_ext.h``) name for name; ``runner`` strings one step
together (build on the host, copy the metadata, rope + append, attention) on a torch stream.
libcb.so must be built first (``python -m chunked_prefill_mixed_decode_amd.build``); every entry
point raises ImportError if it is missing.  There is no CPU fallback.
"""
from . import binding  # noqa: F401
