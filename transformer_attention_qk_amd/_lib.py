"""ctypes loader for libattn.so (the C ABI declared in include/attn.h).

Argument marshalling only: no arithmetic of the method happens in Python. Loading fails loudly
when the library has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

c_int, c_float, c_double, c_void_p, c_char_p = (ctypes.c_int, ctypes.c_float, ctypes.c_double,
                                                 ctypes.c_void_p, ctypes.c_char_p)
c_int_p = ctypes.POINTER(ctypes.c_int)

# name -> (restype, argtypes); mirrors include/attn.h
SIGNATURES = {
    "attn_strerror": (c_char_p, [c_int]),
    "attn_version": (c_int, []),
    "attn_sssl_windows": (c_int, [c_int, c_int, c_char_p, c_int_p]),
    "attn_rope_table": (c_int, [c_void_p, c_void_p, c_int, c_int, c_double, c_void_p]),
    "attn_qknorm_rope": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_int, c_int, c_int, c_int, c_float, c_int, c_void_p]),
    "attn_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                         c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p]),
    "attn_fwd_qnorm": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_int, c_int, c_int, c_int, c_float, c_int, c_int,
                               c_int, c_void_p]),
    "attn_fwd_qknorm": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_float,
                                c_int, c_int, c_int, c_void_p]),
    "attn_qknorm_rope_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_int,
                                    c_void_p]),
    "attn_fwd_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                            c_void_p]),
    "attn_fwd_qnorm_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_float,
                                  c_int, c_int, c_int, c_void_p]),
    "attn_fwd_qknorm_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                                   c_float, c_int, c_int, c_int, c_void_p]),
    "attn_bwd": (c_int, [c_void_p] * 10 + [c_int] * 7 + [c_void_p]),
    "attn_bwd_ex": (c_int, [c_void_p] * 10 + [c_int] * 9 + [c_void_p]),
    "attn_qknorm_rope_bwd": (c_int, [c_void_p] * 8 + [c_int] * 4 + [c_float, c_int, c_void_p]),
    "attn_qknorm_rope_bwd_ex": (c_int, [c_void_p] * 8 + [c_int] * 6 + [c_float, c_int, c_void_p]),
    "attn_value_gate_ex": (c_int, [c_void_p] * 4 + [c_int] * 6 + [c_void_p]),
    "attn_fwd_qknorm_ve_ex": (c_int, [c_void_p] * 11 + [c_int] * 6 + [c_float] + [c_int] * 3
                              + [c_void_p]),
    "attn_value_gate_bwd_ex": (c_int, [c_void_p] * 5 + [c_int] * 6 + [c_void_p]),
    "attn_decode_workspace_bytes": (ctypes.c_longlong, [c_int] * 5),
    "attn_decode": (c_int, [c_void_p] * 7 + [ctypes.c_longlong] + [c_int] * 6 + [c_void_p]),
    "attn_decode_ex": (c_int, [c_void_p] * 7 + [ctypes.c_longlong] + [c_int] * 8 + [c_void_p]),
    "attn_decode_noalloc_ex": (c_int, [c_void_p] * 6 + [c_int] * 8 + [c_void_p]),
}

# storage orders (attn_layout)
ATTN_LAYOUT_BHTD = 0
ATTN_LAYOUT_BTHD = 1

# status codes (include/attn.h)
ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_HEAD_DIM = 3
ATTN_ERR_DTYPE = 4
ATTN_ERR_ALIGN = 5
ATTN_ERR_WINDOW = 6
ATTN_ERR_ALIAS = 7
ATTN_ERR_ARG = 8
ATTN_ERR_HIP = 9
ATTN_ERR_SCRATCH = 10

# fixed device scratch of attn_decode_noalloc_ex (ATTN_DECODE_SCRATCH_BYTES)
ATTN_DECODE_SCRATCH_BYTES = 8 << 20

ATTN_BF16 = 0
ATTN_F32 = 1

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open libattn.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m transformer_attention_qk_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class AttnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        msg = load().attn_strerror(code).decode()
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def check(fn: str, code: int) -> None:
    if code != ATTN_OK:
        raise AttnError(fn, code)
