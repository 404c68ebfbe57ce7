"""ctypes loader for libwush.so (the C ABI declared in include/wush.h).

The library is loaded from this package directory.  There is no fallback:
if it has not been built, importing the ops raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwush.so")

WUSH_OK, WUSH_EINVAL, WUSH_EALIGN, WUSH_EUNSUPPORTED, WUSH_EHIP = range(5)
FMT = {"mxfp4": 0, "nvfp4": 1, "int4": 2}

# name -> (restype, argtypes); every entry point declared in include/wush.h
_c_int, _i64, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
SIGNATURES = {
    "wush_quant_mxfp4": (_c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "wush_quant_nvfp4": (_c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "wush_quant_int4": (_c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "wush_quant": (_c_int, [_c_int, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "wush_gemm_mxfp4": (_c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _c_int, _vp]),
    "wush_gemm_mxfp4_packed": (_c_int, [_vp, _vp, _c_int, _vp, _vp, _i64, _i64, _i64, _vp, _c_int, _vp]),
    "wush_quant_mxfp4_packed": (_c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "wush_gemm_pack_b": (_c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "wush_dequant": (_c_int, [_c_int, _vp, _vp, _vp, _i64, _i64, _vp, _vp]),
    "wush_gptq_block": (_c_int, [_c_int, _vp, _vp, _c_int, _i64, _vp, _vp, _i64, _vp, _i64, _vp]),
    "wush_gptq_wush": (_c_int, [_c_int, _vp, _vp, _i64, _i64, _i64, _c_int, ctypes.c_double, _c_int, _vp, _vp, _vp,
                                _vp, _vp, _vp, _vp]),
    "wush_build_transforms": (_c_int, [_vp, _i64, _vp, _i64, _i64, _c_int, ctypes.c_double, _c_int, _vp, _vp, _vp,
                                       _vp, _vp]),
    "wush_transform_f32": (_c_int, [_vp, _vp, _i64, _i64, _c_int, _vp, _vp]),
    "wush_absmax_transformed": (_c_int, [_vp, _vp, _i64, _i64, _c_int, _vp, _vp]),
    "wush_fixed_transforms": (_c_int, [_c_int, _i64, _c_int, _vp, _vp, _vp]),
    "wush_f64_to_bf16": (_c_int, [_vp, _i64, _vp, _vp]),
    "wush_nvfp4_global_scale": (_c_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "wush_e2m1_encode": (_c_int, [_vp, _i64, _vp, _vp]),
    "wush_status_string": (ctypes.c_char_p, [_c_int]),
    "wush_last_error": (ctypes.c_char_p, []),
    "wush_abi_version": (_c_int, []),
}

ABI_VERSION = 2


class WushError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__("%s failed: status %d (%s)" % (where, status, detail))
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libwush.so once; raise if it is missing or has the wrong ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libwush.so is not built (%s); run `python -m mxfp4_activation_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.wush_abi_version() != ABI_VERSION:
        raise ImportError("libwush.so ABI version mismatch")
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != WUSH_OK:
        lib = load()
        detail = lib.wush_last_error().decode() or lib.wush_status_string(status).decode()
        raise WushError(status, where, detail)
