"""ctypes loader for libvit.so.

The library is built in-tree by ``vision_encoder_varlen_amd.build`` (or
``__graft_entry__.build()``).  Loading fails loudly when it is missing: there is
no fallback implementation of any kind.
"""
from __future__ import annotations

import ctypes
import os
import threading

# VIT_LIBRARY names another build of the same library to load instead (the
# host-sanitizer build the CPU tests use); it must export the same C ABI.
LIB_PATH = os.environ.get("VIT_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libvit.so")

VIT_OK = 0
VIT_ERR_INVALID_ARG = 1
VIT_ERR_UNSUPPORTED = 2
VIT_ERR_HIP = 3
VIT_F32 = 0
VIT_BF16 = 1
VIT_ROPE_NEOX = 0
VIT_ROPE_COMPLEX = 1
VIT_ATTN_CAUSAL = 1

# (name, restype, argtypes) of every function include/vit.h declares.
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
SIGNATURES = {
    "vit_qk_norm_rope": (_I, [_P, _P, _I64, _I, _I, _I, _P, _F, _P, _P, _F, _P]),
    "vit_qk_norm_rope_strided": (_I, [_P, _P, _I64, _I, _I, _I, _P, _F, _P, _P, _F, _P, _P]),
    "vit_qk_norm_rope_ex": (_I, [_P, _P, _I64, _I, _I, _I, _P, _F, _P, _P, _F, _I, _P, _P]),
    "vit_qk_norm_rope_worklist": (_I, [_P, _P, _I64, _I, _I, _I, _P, _F, _P, _P, _F, _I, _P,
                                       _P, _I, _I, _I, _P, _I64, _P, _P]),
    "vit_qk_norm_rope_into": (_I, [_P, _P, _P, _P, _P, _I64, _I, _I, _I, _P, _F, _P, _P, _F, _I,
                                   _P, _P, _I, _I, _I, _P, _I64, _P, _P]),
    "vit_varlen_attn": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P]),
    "vit_varlen_attn_f32": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P]),
    "vit_attn_block_m": (_I, [_I, _I, _I]),
    "vit_worklist_capacity": (_I64, [_I, _I, _I]),
    "vit_varlen_worklist": (_I, [_P, _I, _I, _I, _P, _I64, _P, _P]),
    "vit_varlen_attn_planned": (_I, [_P, _P, _P, _P, _P, _I64, _P, _I, _I, _F, _I, _I, _P, _P, _P,
                                     _P]),
    "vit_varlen_attn_ex": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P, _P]),
    "vit_varlen_attn_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P, _P]),
    "vit_varlen_attn_planned_qnorm_rope": (_I, [_P, _P, _P, _P, _P, _I64, _P, _I, _I, _F, _I, _I,
                                                _P, _F, _P, _F, _I, _P, _P, _P, _P]),
    "vit_varlen_attn_planned_qk_norm_rope": (_I, [_P, _P, _P, _P, _P, _I64, _P, _I, _I, _F, _I,
                                                  _I, _P, _F, _P, _P, _F, _I, _P, _P, _P, _P]),
    "vit_varlen_attn_strided": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P]),
    "vit_dense_batch_attn": (_I, [_P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P, _P]),
    "vit_varlen_attn_lse": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _P]),
    "vit_device_error": (_I, [_P, ctypes.POINTER(ctypes.c_int32), _I]),
    "vit_time_next_kernel": (_I, [_P, _P]),
    "vit_last_error": (ctypes.c_char_p, []),
    "vit_release": (None, []),
}

_lock = threading.Lock()
_lib = None


class VitError(ValueError):
    """A libvit.so call returned a nonzero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libvit status {status}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


# The MFMA-rate probe (measurement support) lives in a library of its own.
PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvit_probe.so")
PROBE_SIGNATURES = {
    "vit_probe_mfma": (_I, [_P, _I64, _I, _I, _P, _P]),
    "vit_probe_last_error": (ctypes.c_char_p, []),
}
_probe = None


def load_probe() -> ctypes.CDLL:
    global _probe
    with _lock:
        if _probe is not None:
            return _probe
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is missing: build the HIP libraries first")
        lib = ctypes.CDLL(PROBE_PATH)
        for name, (res, args) in PROBE_SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _probe = lib
        return lib


def check(status: int) -> None:
    if status != VIT_OK:
        msg = load().vit_last_error().decode("utf-8", "replace")
        raise VitError(status, msg)
