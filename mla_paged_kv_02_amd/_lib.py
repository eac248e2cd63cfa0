"""ctypes loader for libmla_paged_kv.so (the C ABI in include/mla_paged_kv.h).

The library is built in-tree by mla_paged_kv_02_amd.build.  Loading fails
loudly when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_paged_kv.so")

# exported symbols, in header order
SYMBOLS = ("mla_status_str", "mla_last_error", "mla_device_cus", "mla_default_num_parts",
           "mla_metadata_ints", "mla_workspace_bytes", "mla_get_metadata", "mla_decode",
           "mla_decode_noalloc", "mla_combine", "mla_absorb_bmm", "mla_absorb_bmm_fp8w", "mla_probe_read",
           "mla_probe_mfma", "mla_probe_lds")

MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE = 3
MLA_ERR_HIP = 4
# bytes of the scratch array mla_decode_noalloc uses on each device
NOALLOC_SCRATCH_BYTES = 160 << 20

_lib = None


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, status_str(status), detail))


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmla_paged_kv.so is not built (expected at %s); run "
                           "`python -m mla_paged_kv_02_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.mla_status_str.restype = ctypes.c_char_p
    lib.mla_status_str.argtypes = [i32]
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_device_cus.restype = i32
    lib.mla_device_cus.argtypes = [i32, ctypes.POINTER(ctypes.c_int)]
    lib.mla_default_num_parts.restype = i32
    lib.mla_default_num_parts.argtypes = [i32, i32, i32, i32]
    lib.mla_metadata_ints.restype = sz
    lib.mla_metadata_ints.argtypes = [i32, i32]
    lib.mla_workspace_bytes.restype = sz
    lib.mla_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.mla_get_metadata.restype = i32
    lib.mla_get_metadata.argtypes = [P, i32, i32, i32, i32, P, P]
    lib.mla_decode.restype = i32
    lib.mla_decode.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, i32, i32, i32,
                               ctypes.c_float, i32, P, i32, P, sz, P, P, P]
    lib.mla_decode_noalloc.restype = i32
    lib.mla_decode_noalloc.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_float, i32, P, i32, P, P, P]
    lib.mla_combine.restype = i32
    lib.mla_combine.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P]
    lib.mla_absorb_bmm.restype = i32
    lib.mla_absorb_bmm.argtypes = [P, i64, i64, P, i32, i32, i32, P, i64, i64, i32, P]
    lib.mla_absorb_bmm_fp8w.restype = i32
    lib.mla_absorb_bmm_fp8w.argtypes = [P, i64, i64, P, P, i32, i32, i32, P, i64, i64, i32, P]
    lib.mla_probe_read.restype = i32
    lib.mla_probe_read.argtypes = [P, i64, i32, P, P]
    lib.mla_probe_mfma.restype = i32
    lib.mla_probe_mfma.argtypes = [i32, i32, P, P]
    lib.mla_probe_lds.restype = i32
    lib.mla_probe_lds.argtypes = [i32, i32, i32, i32, P, P, P]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().mla_status_str(int(status)).decode()


def last_error() -> str:
    return load().mla_last_error().decode()


def check(status: int, where: str) -> None:
    if status != MLA_OK:
        raise MlaError(status, where, last_error())
