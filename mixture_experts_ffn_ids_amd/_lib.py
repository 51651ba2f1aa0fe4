"""ctypes loader for libmoe.so (the C ABI declared in include/moe.h).

Loading fails loudly when the library has not been built: there is no other
implementation of the layer in this package.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
                4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_BAD_ID", 6: "MOE_ERR_DUP_ID", 7: "MOE_ERR_HIP",
                8: "MOE_ERR_DEVICE"}

FLAG_CHECKED = 1
FLAG_TILE_16 = 1 << 4
FLAG_TILE_128 = 2 << 4
FLAG_TILE_192 = 3 << 4
FLAG_TILE_256 = 4 << 4
FLAG_TILE_224 = 5 << 4

KERNEL_QUANT, KERNEL_DISPATCH, KERNEL_GATE_UP, KERNEL_DOWN, KERNEL_COMBINE = range(5)


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        msg = f"{where}: {self.name} ({_lib_handle().moe_status_string(status).decode()})"
        if status == 7:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


_handle = None


def _lib_handle():
    global _handle
    if _handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m mixture_experts_ffn_ids_amd.build` "
                "(the layer has no implementation other than the HIP library)")
        lib = ctypes.CDLL(LIB_PATH)
        P, i64, i32, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        st = ctypes.c_int
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_last_hip_error.restype = ctypes.c_int
        lib.moe_last_hip_error.argtypes = []
        lib.moe_dispatch_workspace_size.restype = sz
        lib.moe_dispatch_workspace_size.argtypes = [i64, i32, i32]
        lib.moe_dispatch.restype = st
        lib.moe_dispatch.argtypes = [P, i64, i32, i32, P, P, P, P, P, sz, u32, P]
        lib.moe_swiglu_workspace_size.restype = sz
        lib.moe_swiglu_workspace_size.argtypes = [i64, i32, i32, i32, i32]
        lib.moe_grouped_swiglu.restype = st
        lib.moe_grouped_swiglu.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, sz, u32, P]
        lib.moe_combine.restype = st
        lib.moe_combine.argtypes = [P, P, P, P, i64, i32, i32, P, P]
        lib.moe_combine_residual.restype = st
        lib.moe_combine_residual.argtypes = [P, P, P, P, P, i64, i32, i32, P, P]
        lib.moe_swiglu_q_workspace_size.restype = sz
        lib.moe_swiglu_q_workspace_size.argtypes = [i64, i32, i32, i32, i32]
        lib.moe_grouped_swiglu_q.restype = st
        lib.moe_grouped_swiglu_q.argtypes = [P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, sz, u32, P]
        lib.moe_grouped_swiglu_top1.restype = st
        lib.moe_grouped_swiglu_top1.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, sz, u32,
                                                P]
        lib.moe_grouped_swiglu_noalloc.restype = st
        lib.moe_grouped_swiglu_noalloc.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, u32, P]
        lib.moe_rmsnorm_quantize_rows.restype = st
        lib.moe_rmsnorm_quantize_rows.argtypes = [P, P, ctypes.c_float, i64, i32, P, P, P, P]
        lib.moe_quantize_rows.restype = st
        lib.moe_quantize_rows.argtypes = [P, i64, i32, P, P, P]
        lib.moe_profile_enable.restype = st
        lib.moe_profile_enable.argtypes = [ctypes.c_int]
        lib.moe_profile_enable_kinds.restype = st
        lib.moe_profile_enable_kinds.argtypes = [ctypes.c_uint32]
        lib.moe_profile_reset.restype = st
        lib.moe_profile_reset.argtypes = []
        lib.moe_profile_read.restype = st
        lib.moe_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        _handle = lib
    return _handle


def lib():
    return _lib_handle()


def check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where, _lib_handle().moe_last_hip_error())
