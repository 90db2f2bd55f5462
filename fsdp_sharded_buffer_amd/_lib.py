"""ctypes declarations of librs.so (include/rs.h).  Loads the in-tree
library and fails loudly when it has not been built."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librs.so")


class rs_tensor_spec(ctypes.Structure):
    _fields_ = [("rows", c_int64), ("cols", c_int64), ("gran_rows", c_int64),
                ("q_rows", c_int32), ("q_cols", c_int32)]


class rs_plan_info(ctypes.Structure):
    _fields_ = [("S", c_int64), ("total", c_int64), ("numel", c_int64), ("pad_elems", c_int64),
                ("pad_frac", c_double), ("lower_bound", c_int64), ("peak_param_bytes", c_int64),
                ("seconds", c_double)]


class rs_layout_info(ctypes.Structure):
    _fields_ = [("n", c_int32), ("m", c_int32), ("S", c_int64), ("total", c_int64),
                ("num_chunks", c_int64), ("num_coarse_chunks", c_int64), ("num_frags", c_int64), ("num_tiles", c_int64),
                ("chunk_elems", c_int64), ("device_bytes", c_int64), ("workspace_bytes", c_int64)]


class rs_adamw_params(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("bias_correction1", c_float),
                ("bias_correction2", c_float), ("grad_scale", c_float)]


class rs_sgd_params(ctypes.Structure):
    _fields_ = [("lr", c_float), ("momentum", c_float), ("weight_decay", c_float),
                ("grad_scale", c_float), ("nesterov", c_int32)]


class RsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"rs status {status}: {msg}")
        self.status = status


# name -> (restype, argtypes); every entry point declared in include/rs.h
SIGNATURES = {
    "rs_plan": (c_int32, [POINTER(rs_tensor_spec), c_int32, c_int32, c_int64, c_int64,
                          POINTER(c_int64), POINTER(rs_plan_info)]),
    "rs_plan_order": (c_int32, [POINTER(rs_tensor_spec), c_int32, c_int32, POINTER(c_int32)]),
    "rs_plan_ordered": (c_int32, [POINTER(rs_tensor_spec), c_int32, c_int32, c_int64, c_int64,
                                  c_int32, POINTER(c_int32), POINTER(c_int64),
                                  POINTER(rs_plan_info)]),
    "rs_layout_create": (c_int32, [POINTER(rs_tensor_spec), c_int32, c_int32, c_int64,
                                   POINTER(c_int64), c_int64, POINTER(c_void_p)]),
    "rs_layout_get_info": (c_int32, [c_void_p, POINTER(rs_layout_info)]),
    "rs_layout_upload": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "rs_layout_destroy": (None, [c_void_p]),
    "rs_layout_device_bytes": (c_size_t, [c_void_p]),
    "rs_workspace_bytes": (c_size_t, [c_void_p]),
    "rs_pack": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32,
                          c_void_p]),
    "rs_unpack": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32,
                            c_void_p]),
    "rs_group_scale_add": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_float, c_float,
                                     c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
    "rs_group_zero": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32,
                                c_void_p]),
    "rs_ragged_sqnorm": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_int32, c_int32, c_void_p]),
    "rs_ragged_sqnorm_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_int32, c_int32, c_void_p]),
    "rs_block_quant": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                 c_int32, c_int32, c_void_p]),
    "rs_block_dequant": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                   c_int32, c_int32, c_void_p]),
    "rs_adamw_step": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                POINTER(rs_adamw_params), c_void_p, c_void_p, c_int32, c_int32,
                                c_void_p]),
    "rs_adamw8_step": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_int32, POINTER(rs_adamw_params), c_void_p, c_int32,
                                 c_int32, c_void_p]),
    "rs_sgd_step": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, POINTER(rs_sgd_params),
                              c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
    "rs_status_str": (c_char_p, [c_int32]),
    "rs_last_error": (c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m fsdp_sharded_buffer_amd.build` "
                               "(there is no CPU fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise RsError(status, lib().rs_last_error().decode())
