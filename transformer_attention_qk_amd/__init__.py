"""MI355X (gfx950) QK-RMSNorm + RoPE + causal / sliding-window attention forward.

The compute lives in ``libattn.so`` (hand-written HIP kernels behind a C ABI declared in
``include/attn.h``); :mod:`.ops` is a thin ctypes binding over it. Importing this package loads
nothing; the library is opened on first use.
"""

__all__ = ["inputs", "ops"]
