"""ctypes binding of libint8lin.so (argument marshalling only).

Every computation runs in the library's HIP kernels; torch provides device
memory (outputs and workspaces are allocated with torch.empty) and the current
stream.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libint8lin.so")

I8L_OK = 0
STATUS_NAMES = {
    0: "I8L_OK",
    1: "I8L_ERR_INVALID_ARG",
    2: "I8L_ERR_K_TOO_LARGE",
    3: "I8L_ERR_WORKSPACE",
    4: "I8L_ERR_HIP",
}
MAX_K = 133136
MAX_K_ZP = 66304
STATIC_SCRATCH_BYTES = 32 << 20   # I8L_STATIC_SCRATCH_BYTES

# Every symbol include/int8lin.h declares.
EXPORTS = (
    "i8l_linear_workspace",
    "i8l_linear_workspace_bytes",
    "int8_quantize_weight",
    "int8_linear",
    "int8_linear_bias",
    "int8_linear_static",
    "int8_quantize_activation",
    "int8_gemm_i32",
    "int8_weight_code_sums",
    "int8_linear_zp",
    "int8_quantize_activation_zp",
    "i8l_backward_weight_workspace_bytes",
    "int8_linear_backward_input",
    "int8_linear_backward_weight",
    "i8l_last_error",
    "i8l_build_info",
)


class Int8LinError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [
        ("total", ctypes.c_size_t),
        ("n_outliers", ctypes.c_size_t),
        ("outlier_idx", ctypes.c_size_t),
        ("sx", ctypes.c_size_t),
        ("Xq", ctypes.c_size_t),
        ("X_outliers", ctypes.c_size_t),
        ("flags", ctypes.c_size_t),
        ("gemm_counters", ctypes.c_size_t),
        ("gemm_partials", ctypes.c_size_t),
        ("gemm_slices", ctypes.c_size_t),
        ("zero_points", ctypes.c_size_t),
        ("act_partials", ctypes.c_size_t),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m mixed_precision_quantized_int8_amd.build` (hipcc, gfx950)"
        )
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.i8l_linear_workspace.argtypes = [i64, i64, i64, ctypes.POINTER(WorkspaceLayout)]
    L.i8l_linear_workspace.restype = ctypes.c_int
    L.i8l_linear_workspace_bytes.argtypes = [i64, i64, i64]
    L.i8l_linear_workspace_bytes.restype = sz
    L.int8_quantize_weight.argtypes = [vp, i64, i64, vp, vp, vp]
    L.int8_quantize_weight.restype = ctypes.c_int
    L.int8_linear.argtypes = [vp, i64, i64, vp, vp, i64, vp, f32, vp, vp, sz, vp]
    L.int8_linear.restype = ctypes.c_int
    L.int8_linear_bias.argtypes = [vp, i64, i64, vp, vp, i64, vp, vp, f32, vp, vp, sz, vp]
    L.int8_linear_bias.restype = ctypes.c_int
    L.int8_linear_static.argtypes = [vp, i64, i64, vp, vp, i64, vp, vp, f32, vp, vp]
    L.int8_linear_static.restype = ctypes.c_int
    L.int8_quantize_activation.argtypes = [vp, i64, i64, f32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.int8_quantize_activation.restype = ctypes.c_int
    L.int8_gemm_i32.argtypes = [vp, vp, i64, i64, i64, vp, vp, sz, vp]
    L.int8_gemm_i32.restype = ctypes.c_int
    L.int8_weight_code_sums.argtypes = [vp, i64, i64, vp, vp]
    L.int8_weight_code_sums.restype = ctypes.c_int
    L.int8_linear_zp.argtypes = [vp, i64, i64, vp, vp, vp, i64, vp, vp, f32, vp, vp, sz, vp]
    L.int8_linear_zp.restype = ctypes.c_int
    L.int8_quantize_activation_zp.argtypes = [vp, i64, i64, f32, vp, vp, vp, vp, vp, vp, vp, sz,
                                              vp]
    L.int8_quantize_activation_zp.restype = ctypes.c_int
    L.i8l_backward_weight_workspace_bytes.argtypes = [i64, i64, i64]
    L.i8l_backward_weight_workspace_bytes.restype = sz
    L.int8_linear_backward_input.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    L.int8_linear_backward_input.restype = ctypes.c_int
    L.int8_linear_backward_weight.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    L.int8_linear_backward_weight.restype = ctypes.c_int
    L.i8l_last_error.argtypes = []
    L.i8l_last_error.restype = ctypes.c_char_p
    L.i8l_build_info.argtypes = []
    L.i8l_build_info.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status: int) -> None:
    if status != I8L_OK:
        raise Int8LinError(status, lib().i8l_last_error().decode())


def last_error() -> str:
    return lib().i8l_last_error().decode()


def build_info() -> str:
    return lib().i8l_build_info().decode()


def workspace_layout(M: int, K: int, N: int = 0) -> dict:
    L = WorkspaceLayout()
    check(lib().i8l_linear_workspace(M, K, N, ctypes.byref(L)))
    return {name: getattr(L, name) for name, _ in WorkspaceLayout._fields_}


def workspace_bytes(M: int, K: int, N: int = 0) -> int:
    return int(lib().i8l_linear_workspace_bytes(M, K, N))
