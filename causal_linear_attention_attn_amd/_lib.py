"""ctypes view of liblinattn.so (include/linattn.h).  Marshalling only."""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblinattn.so")

LA_OK, LA_EINVAL, LA_EUNSUPPORTED, LA_EHIP, LA_EWORKSPACE, LA_ESCRATCH = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 128 << 20  # LA_NOALLOC_SCRATCH_BYTES
LA_F32, LA_BF16 = 0, 1
LA_FMAP_IDENTITY, LA_FMAP_ELU1 = 0, 1
LA_RULE_LINEAR, LA_RULE_DELTA = 0, 1
ABI_VERSION = 7

# Every symbol include/linattn.h declares.
EXPORTS = ("la_prefill_workspace_size", "la_prefill", "la_prefill_noalloc", "la_decode_step",
           "la_backward_workspace_size", "la_backward",
           "la_delta_backward_workspace_size", "la_delta_backward",
           "la_state_init", "la_status_str", "la_abi_version",
           "la_profile_enable", "la_profile_collect")

_i32, _ptr, _f32, _size = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("B", _i32), ("H", _i32), ("N", _i32), ("d", _i32), ("dv", _i32),
        ("dtype", _i32), ("rule", _i32), ("fmap", _i32),
        ("q", _ptr), ("k", _ptr), ("v", _ptr),
        ("gamma", _ptr), ("g", _ptr), ("alpha", _ptr),
        ("conv_weight", _ptr), ("conv_width", _i32), ("conv_in", _ptr), ("conv_out", _ptr),
        ("eps", _f32), ("S_in", _ptr), ("z_in", _ptr), ("S_out", _ptr), ("z_out", _ptr),
        ("o", _ptr), ("den_out", _ptr), ("workspace", _ptr), ("workspace_bytes", _size),
    ]


class BackwardArgs(ctypes.Structure):
    _fields_ = [
        ("B", _i32), ("H", _i32), ("N", _i32), ("d", _i32), ("dv", _i32),
        ("dtype", _i32), ("fmap", _i32),
        ("q", _ptr), ("k", _ptr), ("v", _ptr), ("o", _ptr), ("den", _ptr), ("grad_o", _ptr),
        ("gamma", _ptr), ("S_in", _ptr), ("z_in", _ptr),
        ("grad_S_out", _ptr), ("grad_z_out", _ptr),
        ("grad_q", _ptr), ("grad_k", _ptr), ("grad_v", _ptr),
        ("grad_S_in", _ptr), ("grad_z_in", _ptr),
        ("workspace", _ptr), ("workspace_bytes", _size),
        ("fwd_workspace", _ptr), ("fwd_workspace_bytes", _size),
        ("conv_weight", _ptr), ("conv_width", _i32), ("conv_in", _ptr), ("grad_conv_out", _ptr),
        ("grad_conv_weight", _ptr), ("grad_conv_in", _ptr),
        ("alpha", _ptr), ("grad_alpha", _ptr),
    ]


class DeltaBackwardArgs(ctypes.Structure):
    _fields_ = [
        ("B", _i32), ("H", _i32), ("N", _i32), ("d", _i32), ("dv", _i32), ("dtype", _i32),
        ("q", _ptr), ("k", _ptr), ("v", _ptr), ("g", _ptr), ("alpha", _ptr), ("S_in", _ptr),
        ("grad_o", _ptr), ("grad_S_out", _ptr),
        ("grad_q", _ptr), ("grad_k", _ptr), ("grad_v", _ptr), ("grad_g", _ptr),
        ("grad_alpha", _ptr), ("grad_S_in", _ptr),
        ("workspace", _ptr), ("workspace_bytes", _size),
        ("conv_weight", _ptr), ("conv_width", _i32), ("conv_in", _ptr), ("grad_conv_out", _ptr),
        ("grad_conv_weight", _ptr), ("grad_conv_in", _ptr),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("B", _i32), ("H", _i32), ("d", _i32), ("dv", _i32),
        ("dtype", _i32), ("rule", _i32), ("fmap", _i32),
        ("q", _ptr), ("k", _ptr), ("v", _ptr),
        ("gamma", _ptr), ("g", _ptr), ("alpha", _ptr),
        ("conv_weight", _ptr), ("conv_width", _i32), ("conv_cache", _ptr),
        ("eps", _f32), ("S", _ptr), ("z", _ptr), ("o", _ptr),
    ]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("ms", _f32)]


_lock = threading.Lock()
_lib = None


class LibraryMissing(RuntimeError):
    pass


def load(path: str | None = None):
    """Load the library once (raises LibraryMissing if it was never built)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise LibraryMissing(
                f"{p} is missing: build it with "
                "`python -m causal_linear_attention_attn_amd.build`")
        lib = ctypes.CDLL(p)
        lib.la_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs)]
        lib.la_prefill_workspace_size.restype = _size
        lib.la_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _ptr]
        lib.la_prefill.restype = ctypes.c_int
        lib.la_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), _ptr]
        lib.la_prefill_noalloc.restype = ctypes.c_int
        lib.la_backward_workspace_size.argtypes = [ctypes.POINTER(BackwardArgs)]
        lib.la_backward_workspace_size.restype = _size
        lib.la_backward.argtypes = [ctypes.POINTER(BackwardArgs), _ptr]
        lib.la_backward.restype = ctypes.c_int
        lib.la_delta_backward_workspace_size.argtypes = [ctypes.POINTER(DeltaBackwardArgs)]
        lib.la_delta_backward_workspace_size.restype = _size
        lib.la_delta_backward.argtypes = [ctypes.POINTER(DeltaBackwardArgs), _ptr]
        lib.la_delta_backward.restype = ctypes.c_int
        lib.la_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _ptr]
        lib.la_decode_step.restype = ctypes.c_int
        lib.la_state_init.argtypes = [_ptr, _ptr, _i32, _i32, _i32, _i32, _ptr]
        lib.la_state_init.restype = ctypes.c_int
        lib.la_status_str.argtypes = [ctypes.c_int]
        lib.la_status_str.restype = ctypes.c_char_p
        lib.la_profile_enable.argtypes = [ctypes.c_int]
        lib.la_profile_enable.restype = ctypes.c_int
        lib.la_profile_collect.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int]
        lib.la_profile_collect.restype = ctypes.c_int
        lib.la_abi_version.argtypes = []
        lib.la_abi_version.restype = _i32
        if lib.la_abi_version() != ABI_VERSION:
            raise RuntimeError("liblinattn.so ABI version mismatch; rebuild it")
        if path is None:
            _lib = lib
        return lib


class LinattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load().la_status_str(status).decode()
        super().__init__(f"{where} failed: {msg} (status {status})")
        self.status = status


def check(status: int, where: str):
    if status != LA_OK:
        raise LinattnError(status, where)
