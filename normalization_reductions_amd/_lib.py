"""ctypes declarations of libnormred.so (the C ABI in include/normred.h).

Loading fails loudly: there is no fallback path. If the library has not been built, import of
this module raises with the build command to run.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# NORMRED_LIB selects another build of the same library (the host-sanitizer test loads its
# AddressSanitizer build this way)
LIB_PATH = os.environ.get("NORMRED_LIB") or os.path.join(PKG, "libnormred.so")

NR_OK = 0
NR_ERR_INVALID_ARG = 1
NR_ERR_MISALIGNED = 2
NR_ERR_UNSUPPORTED = 3
NR_ERR_WORKSPACE = 4
NR_ERR_HIP = 5
STATUS_NAMES = {0: "NR_OK", 1: "NR_ERR_INVALID_ARG", 2: "NR_ERR_MISALIGNED",
                3: "NR_ERR_UNSUPPORTED", 4: "NR_ERR_WORKSPACE", 5: "NR_ERR_HIP"}

NR_VARIANT_AUTO = 0
NR_VARIANT_RESIDENT = 1
NR_VARIANT_SPLIT = 2

NR_NORM_BATCH_TRAIN = 1
NR_NORM_INSTANCE = 2


class ConvNormDesc(ctypes.Structure):
    """Mirror of nr_conv_norm_desc."""

    _fields_ = [
        ("spatial_dims", ctypes.c_int32),
        ("ksize", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("C_in", ctypes.c_int64),
        ("C_out", ctypes.c_int64),
        ("in_d", ctypes.c_int64),
        ("in_h", ctypes.c_int64),
        ("in_w", ctypes.c_int64),
        ("norm", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("pre_mul", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("out_scale", ctypes.c_float),
        ("clamp", ctypes.c_int32),
        ("clamp_lo", ctypes.c_float),
        ("clamp_hi", ctypes.c_float),
        ("post_mul", ctypes.c_void_p),
        ("reduce_max_c", ctypes.c_int32),
        ("momentum", ctypes.c_float),
        ("running_mean", ctypes.c_void_p),
        ("running_var", ctypes.c_void_p),
        ("channels_last", ctypes.c_int32),
    ]


# (name, restype, argtypes) for every exported function of normred.h
_vp, _i64, _f, _i, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "nr_last_error": (ctypes.c_char_p, []),
    "nr_version": (ctypes.c_char_p, []),
    "inorm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "inorm_forward": (_i, [_vp, _vp, _i64, _i64, _i64, _f, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "inorm_forward_ex": (_i, [_vp, _vp, _i64, _i64, _i64, _f, _vp, _vp, _vp, _vp, _vp, _sz, _i,
                              _vp]),
    "inorm_forward_noalloc": (_i, [_vp, _vp, _i64, _i64, _i64, _f, _vp, _vp, _vp, _vp, _vp]),
    "bn_train_workspace_size": (_sz, [_i64, _i64, _i64]),
    "bn_train_forward": (_i, [_vp, _vp, _i64, _i64, _i64, _f, _vp, _vp, _f, _vp, _vp, _vp, _sz,
                              _vp]),
    "bn_train_forward_ex": (_i, [_vp, _vp, _i64, _i64, _i64, _f, _vp, _vp, _f, _vp, _vp, _f, _vp,
                                 _vp, _vp, _sz, _vp]),
    "conv_norm_epilogue_workspace_size": (_sz, [ctypes.POINTER(ConvNormDesc)]),
    "conv_norm_epilogue_forward": (_i, [ctypes.POINTER(ConvNormDesc), _vp, _vp, _vp, _vp, _vp,
                                        _sz, _vp]),
    "conv_bn_eval_workspace_size": (_sz, [ctypes.POINTER(ConvNormDesc)]),
    "conv_bn_eval_forward": (_i, [ctypes.POINTER(ConvNormDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _sz, _vp]),
    "nr_workspace_clear": (_i, [_vp, _sz, _vp]),
    "nr_workspace_check": (_i, [_vp, _sz, _vp, ctypes.POINTER(ctypes.c_uint32)]),
    "nr_stream_copy": (_i, [_vp, _vp, _i64, _vp]),
    "nr_stream_copy_ws": (_i, [_vp, _vp, _i64, _vp, _sz, _vp]),
}

_lib = None


def load():
    """Load libnormred.so and declare every signature. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libnormred.so is not built (%s). Build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python normalization_reductions_amd/build.py`." % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    msg = load().nr_last_error()
    return msg.decode() if msg else ""


class NormredError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s: %s" % (where, STATUS_NAMES.get(status, status),
                                                last_error()))


def check(status: int, where: str) -> None:
    if status != NR_OK:
        raise NormredError(status, where)
