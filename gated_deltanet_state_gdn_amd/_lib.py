"""ctypes declarations of the C ABI in include/gdn.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB_PATH selects another build of the same library (e.g. a host-sanitized one)
LIB_PATH = os.environ.get("GDN_LIB_PATH") or os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_UNSUPPORTED = 0, 1, 2, 3, 4
GDN_ERR_ALIGN, GDN_ERR_WORKSPACE, GDN_ERR_LAUNCH, GDN_ERR_DEVICE_INPUT, GDN_ERR_HIP = 5, 6, 7, 8, 9
GDN_ERR_DEVICE_WAIT, GDN_ERR_SCRATCH = 10, 11
GDN_F32, GDN_BF16 = 0, 1
ABI_VERSION = 3

# every symbol include/gdn.h declares
EXPORTS = ("gdn_abi_version", "gdn_status_str", "gdn_replay_len", "gdn_workspace_bytes",
           "gdn_replay", "gdn_prefill", "gdn_state_relerr", "gdn_device_status",
           "gdn_adaptive_replay_len", "gdn_adaptive_replay_len_static",
           "gdn_segmented_workspace_bytes", "gdn_replay_segmented")


class GdnDesc(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("h_qk", ctypes.c_int32), ("h_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32),
                ("o_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("total_tokens", ctypes.c_int64), ("total_out_tokens", ctypes.c_int64)]


class GdnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s: status %d (%s)" % (where, code, status_str(code)))


_lib = None


def load() -> ctypes.CDLL:
    """Load libgdn.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libgdn.so is not built: run `python -m gated_deltanet_state_gdn_amd.build`"
                          " (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    dptr = ctypes.POINTER(GdnDesc)
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = i32
    lib.gdn_status_str.argtypes = [i32]
    lib.gdn_status_str.restype = ctypes.c_char_p
    lib.gdn_replay_len.argtypes = [i32, ctypes.c_double]
    lib.gdn_replay_len.restype = i32
    lib.gdn_workspace_bytes.argtypes = [dptr]
    lib.gdn_workspace_bytes.restype = sz
    lib.gdn_replay.argtypes = [dptr, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_replay.restype = i32
    lib.gdn_prefill.argtypes = [dptr, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_prefill.restype = i32
    lib.gdn_state_relerr.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
    lib.gdn_state_relerr.restype = i32
    lib.gdn_device_status.argtypes = [vp, vp, ctypes.POINTER(i32)]
    lib.gdn_device_status.restype = i32
    lib.gdn_adaptive_replay_len.argtypes = [dptr, vp, vp, ctypes.c_double, i32, i32, vp, vp, sz, vp]
    lib.gdn_adaptive_replay_len.restype = i32
    lib.gdn_adaptive_replay_len_static.argtypes = [dptr, vp, vp, ctypes.c_double, i32, i32, vp, vp]
    lib.gdn_adaptive_replay_len_static.restype = i32
    lib.gdn_segmented_workspace_bytes.argtypes = [dptr, i32]
    lib.gdn_segmented_workspace_bytes.restype = sz
    lib.gdn_replay_segmented.argtypes = [dptr, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.gdn_replay_segmented.restype = i32
    if lib.gdn_abi_version() != ABI_VERSION:
        raise ImportError("libgdn.so ABI version mismatch")
    _lib = lib
    return lib


def status_str(code: int) -> str:
    try:
        return load().gdn_status_str(int(code)).decode()
    except ImportError:
        return "?"
