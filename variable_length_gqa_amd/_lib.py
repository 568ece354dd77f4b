"""ctypes loader for the HIP library ``libvlgqa.so`` (built in-tree by build.py).

There is no fallback: if the library is missing the calls raise.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvlgqa.so")

VLGQA_OK, VLGQA_EINVAL, VLGQA_EUNSUPPORTED, VLGQA_EHIP = 0, 1, 2, 3
VLGQA_F32, VLGQA_F16, VLGQA_BF16 = 0, 1, 2

# (symbol, restype, argtypes) for every entry point in include/vlgqa.h
_P, _I64, _I, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "varlen_attention_fwd": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                  _I64, _I, _I, _P, _P, _P]),
    "flash_attention_fwd": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I, _I64, _I64,
                                 _I, _P, _P, _P]),
    "flash_attention_fwd_fp8": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I, _F, _F,
                                     _F, _F, _P, _P, _P]),
    "flash_attention_decode": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I, _I64,
                                    _I64, _I, _P, _P, _P, _I64, _P]),
    "flash_attention_decode_noalloc": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I,
                                            _I64, _I64, _I, _P, _P, _P]),
    "vlgqa_decode_workspace_floats": (_I64, [_I64, _I64, _I64, _I64]),
    "varlen_attention_bwd": (_I, [_P] * 8 + [_I64] * 8 + [_I, _I] + [_P] * 5),
    "flash_attention_bwd": (_I, [_P] * 6 + [_I64] * 6 + [_I, _I64, _I] + [_P] * 5),
    "flash_attention_bwd_fp8": (_I, [_P] * 6 + [_I64] * 6 + [_I] + [_F] * 8 + [_P] * 4 +
                                [_I64, _P]),
    "vlgqa_bwd_workspace_floats": (_I64, [_I64] * 5 + [_I]),
    "vlgqa_cu_seqlens": (_I, [_P, _I64, _P, _P]),
    "vlgqa_pack": (_I, [_P, _P, _I64, _I64, _I64, _I64, _P, _P]),
    "vlgqa_unpack": (_I, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "vlgqa_last_error": (ctypes.c_char_p, []),
    "vlgqa_version": (ctypes.c_char_p, []),
}

_lib = None


class VlgqaError(RuntimeError):
    """A non-OK return of the C ABI (the code and "argument: reason")."""

    def __init__(self, code: int, message: str):
        super().__init__(f"vlgqa error {code}: {message}")
        self.code = code
        self.message = message


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                              "(run `python -m variable_length_gqa_amd.build`)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(rc: int) -> None:
    if rc != VLGQA_OK:
        msg = load().vlgqa_last_error().decode(errors="replace")
        if rc == VLGQA_EINVAL:
            raise ValueError(f"vlgqa: {msg}")
        raise VlgqaError(rc, msg)
