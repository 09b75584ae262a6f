"""ctypes loader of ``libcfa.so`` (the C ABI in ``include/cfa.h``).

The library is loaded from this package's directory only; there is no fallback. If it is
missing, every call raises: build it with ``python -m causal_flashattention_amd.build``.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcfa.so")

CFA_F32, CFA_BF16, CFA_MXFP8, CFA_MXFP4, CFA_MXFP6, CFA_MXFP6_E3M2 = 0, 1, 2, 3, 4, 5
STATUS = {0: "CFA_OK", 1: "CFA_ERR_NULL", 2: "CFA_ERR_SHAPE", 3: "CFA_ERR_UNSUPPORTED",
          4: "CFA_ERR_ALIGN", 5: "CFA_ERR_WORKSPACE", 6: "CFA_ERR_HIP"}

# every symbol include/cfa.h declares, with its ctypes signature
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "cfa_version": (_I, []),
    "cfa_status_string": (ctypes.c_char_p, [_I]),
    "cfa_last_error": (ctypes.c_char_p, []),
    "cfa_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "cfa_saved_bytes": (_S, [_I, _I, _I, _I, _I, _I]),
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P, _S, _P]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                      _P, _S, _P]),
    "mx_quantize": (_I, [_P, _I, _I, _I, _P, _P, _I, _I, _P, _P, _I, _P, _S, _P]),
    "mx_quantize_fp4": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "mx_quantize_fp6": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "mx_quantize_fp6_e3m2": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "mx_padded_tokens": (_I, [_I, _I]),
    "mx_workspace_bytes": (_S, [_I]),
    "mx_quantize_bytes": (_S, [_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "cfa_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I]),
    "attn_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "cfa_cross_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_fwd_cross": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "attn_bwd_cross": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                            _P, _S, _P]),
    "cfa_set_kernel_events": (_I, [_P, _I]),
    "cfa_device_error": (_I, [_P, _P, ctypes.POINTER(ctypes.c_int)]),
    "attn_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                              _P]),
}

_lib = None


class CfaError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.name}: {detail}")


def lib():
    """The loaded library (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} not found: run `python -m causal_flashattention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status):
    if status != 0:
        raise CfaError(status, lib().cfa_last_error().decode(errors="replace"))
