"""ctypes view of libmoe355.so (include/moe355.h). Marshalling only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe355.so")

MOE_OK = 0
MOE_ERR_INVALID = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_HIP = 3
MOE_ERR_TIMEOUT = 4

MOE_BF16 = 0
MOE_FP8_E4M3_G128 = 1
MOE_MXFP4 = 2

MOE_WEIGHTS_ROW_MAJOR = 0
MOE_WEIGHTS_MFMA_TILED = 1

STATUS_NAMES = {
    MOE_OK: "MOE_OK",
    MOE_ERR_INVALID: "MOE_ERR_INVALID",
    MOE_ERR_UNSUPPORTED: "MOE_ERR_UNSUPPORTED",
    MOE_ERR_HIP: "MOE_ERR_HIP",
    MOE_ERR_TIMEOUT: "MOE_ERR_TIMEOUT",
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}")


class PlanT(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("expert_begin", ctypes.c_int32),
        ("E_local", ctypes.c_int32),
        ("tile", ctypes.c_int32),
        ("rows_cap", ctypes.c_int32),
        ("counts", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p),
        ("pos", ctypes.c_void_p),
        ("src", ctypes.c_void_p),
        ("tile_expert", ctypes.c_void_p),
        ("num_tiles", ctypes.c_void_p),
        ("tile_ready", ctypes.c_void_p),
    ]


class TileConfig(ctypes.Structure):
    _fields_ = [
        ("block_n", ctypes.c_int32),
        ("gemm_workgroups", ctypes.c_int32),
        ("spin_timeout_us", ctypes.c_uint32),
        ("unit_order", ctypes.c_int32),
        ("weight_layout", ctypes.c_int32),
        ("a_stages", ctypes.c_int32),
        ("dispatch_cus", ctypes.c_int32),
        ("unit_rows", ctypes.c_int32),
    ]


# (name, restype, argtypes) of every exported function
_I32, _U32, _SZ, _VP = ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p
_PP = ctypes.POINTER(PlanT)
SIGNATURES = [
    ("moe_pool_rows_upper_bound", _SZ, [_I32, _I32, _I32, _I32]),
    ("moe_workspace_bytes", _SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    ("moe_plan", ctypes.c_int, [_VP, _PP, _VP, _SZ, _VP]),
    ("moe_plan_noalloc", ctypes.c_int, [_VP, _PP, _VP]),
    ("moe_query_pool_rows", ctypes.c_int, [_PP, ctypes.POINTER(_I32), _VP]),
    ("moe_dispatch", ctypes.c_int, [_VP, _I32, _I32, _PP, _I32, _VP, _VP, _U32, _VP, _SZ, _VP]),
    ("moe_expert_ffn", ctypes.c_int,
     [_PP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _U32, _VP, _SZ, _VP,
      ctypes.POINTER(TileConfig), _VP]),
    ("moe_expert_ffn_combine", ctypes.c_int,
     [_PP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _U32, _VP, _SZ, _VP, _VP, _VP,
      ctypes.POINTER(TileConfig), _VP]),
    ("moe_expert_ffn_train", ctypes.c_int,
     [_PP, _I32, _VP, _VP, _VP, _I32, _I32, _U32, _VP, _SZ, _VP, _VP, ctypes.POINTER(TileConfig), _VP]),
    ("moe_combine_backward", ctypes.c_int, [_VP, _VP, _VP, _I32, _PP, _I32, _VP, _VP, _U32, _VP, _SZ, _VP]),
    ("moe_expert_ffn_backward", ctypes.c_int,
     [_PP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _U32, _VP, _SZ, _VP, _VP, _VP, ctypes.POINTER(TileConfig),
      _VP]),
    ("moe_dispatch_backward", ctypes.c_int, [_VP, _I32, _PP, _I32, _VP, _VP]),
    ("moe_pack_weights_transposed", ctypes.c_int, [_VP, _I32, _I32, _I32, _I32, _VP, _VP]),
    ("moe_combine", ctypes.c_int, [_VP, _I32, _VP, _PP, _I32, _VP, _VP]),
    ("moe_pack_weights", ctypes.c_int, [_VP, _I32, _I32, _I32, _I32, _VP, _VP]),
    ("moe_pack_mx_scales", ctypes.c_int, [_VP, _I32, _I32, _I32, _VP, _VP]),
    ("moe_calibrate_mfma", ctypes.c_int, [_I32, _VP, _I32, _VP]),
    ("moe_calibrate_stream", ctypes.c_int, [_VP, _VP, ctypes.c_int64, _I32, _VP, _I32, _VP]),
    ("moe_get_error", ctypes.c_int, [_VP, _SZ, _VP]),
    ("moe_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("moe_device_cu_count", ctypes.c_int, []),
]

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m combine_moe_dispatch_02_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
