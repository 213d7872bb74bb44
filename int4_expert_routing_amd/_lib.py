"""ctypes loader for libmoe_q4.so: argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI declared in
include/moe_q4.h. When the shared library is missing this module raises; there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoe_q4.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGN = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_UNSUPPORTED = -5
MOE_ERR_HIP = -6

MOE_EPI_STORE_F32 = 0
MOE_EPI_SWIGLU_BF16 = 1

MOE_Q4_GROUP = 64
MOE_GEMM_BLOCK_ROWS = 128
MOE_MAX_EXPERTS = 256
MOE_MAX_TOPK = 32
MOE_WORKSPACE_HEAD_BYTES = 190080
MOE_WORKSPACE_STATUS_OFFSET = 16768
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


class MoeDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("block_rows", ctypes.c_int32)]


MOE_Q4_CANONICAL = 0
MOE_Q4_PREPACKED = 1


class MoeQ4Weights(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class MoeLayerOptions(ctypes.Structure):
    _fields_ = [("shared_gate", ctypes.c_void_p), ("side_stream", ctypes.c_void_p),
                ("fork_event", ctypes.c_void_p), ("join_event", ctypes.c_void_p),
                ("persistent_decode", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_DIMS = ctypes.POINTER(MoeDims)
_W = ctypes.POINTER(MoeQ4Weights)

# name -> (restype, argtypes); the same set include/moe_q4.h declares
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_workspace_bytes": (_SZ, [_DIMS]),
    "moe_check_dims": (ctypes.c_int, [_DIMS]),
    "moe_max_tiles": (_I32, [_DIMS]),
    "moe_route": (ctypes.c_int, [_P, _P, _DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_q4": (ctypes.c_int, [_P, _I32, _P, _I32, _W, _W, _P, _P, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "moe_gemm_workspace_bytes": (_SZ, [_I32, _I32]),
    "moe_layer_forward": (ctypes.c_int, [_P, _P, _P, _W, _W, _W, _W, _W, _W, _DIMS, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_forward_ex": (ctypes.c_int, [_P, _P, _P, _W, _W, _W, _W, _W, _W, _DIMS, _P, _P, _P, _P, _P, _SZ, _P,
                                            ctypes.POINTER(MoeLayerOptions)]),
    "moe_prepack_q4_bytes": (_SZ, [_I32, _I32, _I32]),
    "moe_prepack_q4": (ctypes.c_int, [_W, _P, _SZ, _W, _P]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _W, _W, _W, _W, _W, _W, _DIMS, _P, _P, _P, _P, _P]),
    "moe_layer_forward_timed": (ctypes.c_int, [_P, _P, _P, _W, _W, _W, _W, _W, _W, _DIMS, _P, _P, _P, _P, _P, _SZ,
                                               _P, ctypes.POINTER(ctypes.c_void_p), _I32]),
    "moe_quantize_q4": (ctypes.c_int, [_P, ctypes.c_int64, _I32, _P, _P, _P, _P]),
}

MOE_LAYER_STAGE_EVENTS = 6

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python -m int4_expert_routing_amd.build_lib")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)
