"""MI355X-native quantized KV cache: WUSH-KV-style write path and decode attention.

The compute runs in libkvq.so (hand-written HIP kernels for gfx950); this package holds
the ctypes binding (api), the host-side key-transform calibration (calib) and seeded
synthetic input generators (synth)."""
from . import api, calib, synth  # noqa: F401

__all__ = ["api", "calib", "synth"]
