"""ctypes view of libkvstore.so (the C ABI declared in include/kvstore.h).

This module only marshals arguments: it fills ``kvs_tensor`` descriptors from
tensors (or raw pointers), calls the library, and turns non-zero statuses into
exceptions.  All computation happens in the library's HIP kernels; there is no
other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvstore.so")
# the same kernels, the calls first checking the device-resident preconditions
DEBUG_LIB_PATH = os.path.join(_PKG, "libkvstore_debug.so")
# the attention library with the decode kernel's phase timestamps (profiling)
PHASES_LIB_PATH = os.path.join(_PKG, "libkvstore_phases.so")

KVS_OK, KVS_ERR_INVALID, KVS_ERR_UNSUPPORTED, KVS_ERR_WORKSPACE, KVS_ERR_HIP = range(5)
KVS_F32, KVS_BF16, KVS_I32, KVS_FP8_E4M3, KVS_INT8 = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "KVS_OK", 1: "KVS_ERR_INVALID", 2: "KVS_ERR_UNSUPPORTED", 3: "KVS_ERR_WORKSPACE", 4: "KVS_ERR_HIP"}

# every symbol include/kvstore.h declares
EXPORTS = (
    "kv_store_paged",
    "kv_store_rope_paged",
    "kv_store_paged_fp8",
    "attn_varlen_paged_fp8_ex",
    "attn_varlen_paged",
    "attn_varlen_paged_noalloc",
    "attn_varlen_paged_workspace_size",
    "attn_varlen_paged_ex",
    "attn_decode_append_paged",
    "attn_varlen_paged_window_ex",
    "attn_decode_append_paged_window",
    "attn_decode_append_paged_rope",
    "attn_decode_append_paged_fp8",
    "kv_store_paged_int8",
    "attn_varlen_paged_int8_ex",
    "attn_decode_append_paged_int8",
    "kvs_last_error",
    "kvs_last_dispatch",
    "kvs_release_workspace",
)


class KvsTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class KvsHints(ctypes.Structure):
    _fields_ = [
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("decode_tail", ctypes.c_int32),
    ]


KVS_ROPE_NEOX, KVS_ROPE_INTERLEAVED = 0, 1


class KvsRope(ctypes.Structure):
    _fields_ = [
        ("rotary_dim", ctypes.c_int32),
        ("style", ctypes.c_int32),
        ("base", ctypes.c_double),
        ("pos_scale", ctypes.c_double),
    ]


class KvsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def load(path: str = None):
    """Load (once) and return the library (the debug build when the
    environment sets KVS_DEBUG=1).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = DEBUG_LIB_PATH if os.environ.get("KVS_DEBUG") == "1" else LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m attention_kv_store_amd.build); there is no non-HIP implementation")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(KvsTensor)
    vp, st = ctypes.c_void_p, ctypes.c_int
    lib.kv_store_paged.argtypes = [P, P, P, P, P, vp]
    lib.kv_store_paged.restype = st
    lib.kv_store_rope_paged.argtypes = [P, P, P, P, P, P, P, ctypes.POINTER(KvsRope), vp]
    lib.kv_store_rope_paged.restype = st
    lib.kv_store_paged_fp8.argtypes = [P, P, P, P, P, P, P, vp]
    lib.kv_store_paged_fp8.restype = st
    lib.attn_varlen_paged_fp8_ex.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int, ctypes.c_int32,
                                             P, P, ctypes.POINTER(KvsHints), vp, ctypes.c_size_t, vp]
    lib.attn_varlen_paged_fp8_ex.restype = st
    lib.attn_varlen_paged.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, vp]
    lib.attn_varlen_paged.restype = st
    lib.attn_varlen_paged_noalloc.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, vp]
    lib.attn_varlen_paged_noalloc.restype = st
    lib.attn_varlen_paged_workspace_size.argtypes = [P, P, P, ctypes.POINTER(KvsHints)]
    lib.attn_varlen_paged_workspace_size.restype = ctypes.c_size_t
    lib.attn_varlen_paged_ex.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P,
                                         ctypes.POINTER(KvsHints), vp, ctypes.c_size_t, vp]
    lib.attn_varlen_paged_ex.restype = st
    lib.attn_decode_append_paged.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, P, P,
                                             ctypes.POINTER(KvsHints), vp, ctypes.c_size_t, vp]
    lib.attn_decode_append_paged.restype = st
    lib.attn_varlen_paged_window_ex.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_int32, P, P,
                                                ctypes.POINTER(KvsHints), vp, ctypes.c_size_t, vp]
    lib.attn_varlen_paged_window_ex.restype = st
    lib.attn_decode_append_paged_window.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int32, P, P,
                                                    ctypes.POINTER(KvsHints), vp, ctypes.c_size_t, vp]
    lib.attn_decode_append_paged_window.restype = st
    lib.attn_decode_append_paged_rope.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int32,
                                                  ctypes.POINTER(KvsRope), P, P, ctypes.POINTER(KvsHints), vp,
                                                  ctypes.c_size_t, vp]
    lib.attn_decode_append_paged_rope.restype = st
    lib.attn_decode_append_paged_fp8.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int32, P, P,
                                                 ctypes.POINTER(KvsHints), vp, ctypes.c_size_t, vp]
    lib.attn_decode_append_paged_fp8.restype = st
    lib.kv_store_paged_int8.argtypes = lib.kv_store_paged_fp8.argtypes
    lib.kv_store_paged_int8.restype = st
    lib.attn_varlen_paged_int8_ex.argtypes = lib.attn_varlen_paged_fp8_ex.argtypes
    lib.attn_varlen_paged_int8_ex.restype = st
    lib.attn_decode_append_paged_int8.argtypes = lib.attn_decode_append_paged_fp8.argtypes
    lib.attn_decode_append_paged_int8.restype = st
    lib.kvs_last_error.argtypes = []
    lib.kvs_last_error.restype = ctypes.c_char_p
    lib.kvs_last_dispatch.argtypes = []
    lib.kvs_last_dispatch.restype = ctypes.c_char_p
    lib.kvs_release_workspace.argtypes = []
    lib.kvs_release_workspace.restype = st
    _lib = lib
    return lib


def describe(data: int, dtype: int, shape: Sequence[int], strides: Optional[Sequence[int]] = None) -> KvsTensor:
    """A descriptor for raw memory (row-major strides by default)."""
    t = KvsTensor()
    t.data = data
    t.dtype = dtype
    t.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, r) in enumerate(zip(shape, strides)):
        t.shape[i] = int(s)
        t.stride[i] = int(r)
    return t


def check(status: int) -> None:
    if status != KVS_OK:
        raise KvsError(status, load().kvs_last_error().decode())


def last_dispatch() -> str:
    return load().kvs_last_dispatch().decode()
