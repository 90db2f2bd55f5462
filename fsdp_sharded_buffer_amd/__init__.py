"""Python binding of librs.so: RaggedShard flat-buffer planner and grouped
HIP kernels for MI355X (gfx950).

Argument marshalling only: every function forwards to the C entry point of
the same name in include/rs.h.  Tensors may be passed as torch tensors
(their data_ptr() is used) or as raw integer device addresses; `stream`
defaults to torch's current stream on the current device.  There is no CPU
fallback: importing works without a GPU, but every call that launches work
needs the built library and a GPU.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_int64, c_void_p
from typing import Dict, List, Optional, Sequence, Tuple

from ._lib import lib, RsError, check  # noqa: F401
from ._lib import rs_tensor_spec, rs_plan_info, rs_layout_info, rs_adamw_params, rs_sgd_params

RS_F32, RS_BF16, RS_U8 = 0, 1, 2
RS_ERR_NOMEM = -8
RS_Q_FP8_E4M3, RS_Q_INT8 = 0, 1
RS_ORDER_GIVEN, RS_ORDER_BLOCK, RS_ORDER_SHAPE, RS_ORDER_BEST = 0, 1, 2, 3
ORDERS = {"given": RS_ORDER_GIVEN, "block": RS_ORDER_BLOCK, "shape": RS_ORDER_SHAPE,
          "best": RS_ORDER_BEST}

__all__ = [
    "RS_F32", "RS_BF16", "RS_U8", "RS_Q_FP8_E4M3", "RS_Q_INT8", "RsError",
    "RS_ORDER_GIVEN", "RS_ORDER_BLOCK", "RS_ORDER_SHAPE", "RS_ORDER_BEST", "ORDERS",
    "rs_plan", "rs_plan_order", "rs_plan_ordered", "rs_layout_create", "rs_layout_get_info",
    "rs_layout_device_bytes", "rs_workspace_bytes", "rs_layout_upload",
    "rs_layout_destroy", "rs_pack", "rs_unpack", "rs_group_scale_add", "rs_group_zero",
    "rs_ragged_sqnorm", "rs_ragged_sqnorm_noalloc", "rs_block_quant", "rs_block_dequant", "rs_adamw_step", "rs_adamw8_step",
    "rs_sgd_step",
    "rs_status_str", "rs_last_error",
    "Layout", "ptr_table", "dtype_code", "specs_array",
]


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(t) -> int:
    import torch
    return {torch.float32: RS_F32, torch.bfloat16: RS_BF16, torch.uint8: RS_U8}[t.dtype]


def specs_array(specs) -> ctypes.Array:
    """Objects with rows, cols, gran_rows, q_rows, q_cols -> rs_tensor_spec[n]."""
    arr = (rs_tensor_spec * len(specs))()
    for i, s in enumerate(specs):
        arr[i] = rs_tensor_spec(int(s.rows), int(s.cols), int(s.gran_rows),
                                int(getattr(s, "q_rows", 0)), int(getattr(s, "q_cols", 0)))
    return arr


def rs_plan(specs, m: int, align: int = 1, S_cap: int = 0) -> Tuple[List[int], Dict]:
    arr = specs_array(specs)
    offs = (c_int64 * len(specs))()
    info = rs_plan_info()
    check(lib().rs_plan(arr, len(specs), m, align, S_cap, offs, byref(info)))
    return list(offs), {f: getattr(info, f) for f, _ in rs_plan_info._fields_}


def _order_kind(kind) -> int:
    return ORDERS[kind] if isinstance(kind, str) else int(kind)


def rs_plan_order(specs, kind) -> List[int]:
    arr = specs_array(specs)
    perm = (c_int32 * len(specs))()
    check(lib().rs_plan_order(arr, len(specs), _order_kind(kind), perm))
    return list(perm)


def rs_plan_ordered(specs, m: int, align: int = 1, kind="given", S_cap: int = 0
                    ) -> Tuple[List[int], List[int], Dict]:
    """-> (perm, offsets indexed as specs, info)."""
    arr = specs_array(specs)
    perm = (c_int32 * len(specs))()
    offs = (c_int64 * len(specs))()
    info = rs_plan_info()
    check(lib().rs_plan_ordered(arr, len(specs), m, align, S_cap, _order_kind(kind), perm, offs,
                                byref(info)))
    return list(perm), list(offs), {f: getattr(info, f) for f, _ in rs_plan_info._fields_}


def rs_layout_create(specs, m: int, S: int, offsets: Sequence[int], chunk_elems: int = 0) -> c_void_p:
    arr = specs_array(specs)
    offs = (c_int64 * len(specs))(*offsets)
    h = c_void_p()
    check(lib().rs_layout_create(arr, len(specs), m, S, offs, chunk_elems, byref(h)))
    return h


def rs_layout_get_info(layout) -> Dict:
    info = rs_layout_info()
    check(lib().rs_layout_get_info(layout, byref(info)))
    return {f: getattr(info, f) for f, _ in rs_layout_info._fields_}


def rs_layout_device_bytes(layout) -> int:
    return int(lib().rs_layout_device_bytes(layout))


def rs_workspace_bytes(layout) -> int:
    return int(lib().rs_workspace_bytes(layout))


def rs_layout_upload(layout, dev_table, stream=None) -> None:
    check(lib().rs_layout_upload(layout, _ptr(dev_table), _stream(stream)))


def rs_layout_destroy(layout) -> None:
    lib().rs_layout_destroy(layout)


def rs_pack(layout, src, src_dt: int, buf, buf_dt: int, k0: int, k1: int, stream=None) -> None:
    check(lib().rs_pack(layout, _ptr(src), src_dt, _ptr(buf), buf_dt, k0, k1, _stream(stream)))


def rs_unpack(layout, buf, buf_dt: int, dst, dst_dt: int, k0: int, k1: int, stream=None) -> None:
    check(lib().rs_unpack(layout, _ptr(buf), buf_dt, _ptr(dst), dst_dt, k0, k1, _stream(stream)))


def rs_group_scale_add(layout, y, x, x_dt: int, alpha: float, beta: float, tensor_mask=None,
                       found_inf=None, k0: int = 0, k1: int = 1, stream=None) -> None:
    check(lib().rs_group_scale_add(layout, _ptr(y), _ptr(x), x_dt, alpha, beta, _ptr(tensor_mask),
                                   _ptr(found_inf), k0, k1, _stream(stream)))


def rs_group_zero(layout, y, dt: int, tensor_mask=None, k0: int = 0, k1: int = 1, stream=None) -> None:
    check(lib().rs_group_zero(layout, _ptr(y), dt, _ptr(tensor_mask), k0, k1, _stream(stream)))


def rs_ragged_sqnorm(layout, x, sq, partial=None, found_inf=None, ws=None, k0: int = 0, k1: int = 1,
                     stream=None) -> None:
    check(lib().rs_ragged_sqnorm(layout, _ptr(x), _ptr(sq), _ptr(partial), _ptr(found_inf), _ptr(ws),
                                 k0, k1, _stream(stream)))


def rs_ragged_sqnorm_noalloc(layout, x, sq, partial=None, found_inf=None, k0: int = 0,
                             k1: int = 1, stream=None) -> None:
    check(lib().rs_ragged_sqnorm_noalloc(layout, _ptr(x), _ptr(sq), _ptr(partial), _ptr(found_inf),
                                         k0, k1, _stream(stream)))


def rs_block_quant(layout, x, fmt: int, codes, scales, k0: int, k1: int, stream=None,
                   found_inf=None) -> None:
    check(lib().rs_block_quant(layout, _ptr(x), fmt, _ptr(codes), _ptr(scales), _ptr(found_inf),
                               k0, k1, _stream(stream)))


def rs_block_dequant(layout, codes, fmt: int, scales, y, y_dt: int, k0: int, k1: int,
                     stream=None) -> None:
    check(lib().rs_block_dequant(layout, _ptr(codes), fmt, _ptr(scales), _ptr(y), y_dt, k0, k1,
                                 _stream(stream)))


def rs_adamw_step(layout, p, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
                  weight_decay: float, bias_correction1: float, bias_correction2: float,
                  grad_scale: float = 1.0, tensor_mask=None, found_inf=None, k0: int = 0,
                  k1: int = 1, stream=None) -> None:
    hp = rs_adamw_params(lr, beta1, beta2, eps, weight_decay, bias_correction1, bias_correction2,
                         grad_scale)
    check(lib().rs_adamw_step(layout, _ptr(p), _ptr(g), _ptr(m), _ptr(v), byref(hp),
                              _ptr(tensor_mask), _ptr(found_inf), k0, k1, _stream(stream)))


def rs_adamw8_step(layout, p, g, m_codes, m_scales, v_codes, v_scales, fmt: int, lr: float,
                   beta1: float, beta2: float, eps: float, weight_decay: float,
                   bias_correction1: float, bias_correction2: float, grad_scale: float = 1.0,
                   found_inf=None, k0: int = 0, k1: int = 1, stream=None) -> None:
    hp = rs_adamw_params(lr, beta1, beta2, eps, weight_decay, bias_correction1, bias_correction2,
                         grad_scale)
    check(lib().rs_adamw8_step(layout, _ptr(p), _ptr(g), _ptr(m_codes), _ptr(m_scales),
                               _ptr(v_codes), _ptr(v_scales), fmt, byref(hp), _ptr(found_inf),
                               k0, k1, _stream(stream)))


def rs_sgd_step(layout, p, g, buf, lr: float, momentum: float, weight_decay: float,
                nesterov: bool = False, grad_scale: float = 1.0, tensor_mask=None, found_inf=None,
                k0: int = 0, k1: int = 1, stream=None) -> None:
    hp = rs_sgd_params(lr, momentum, weight_decay, grad_scale, 1 if nesterov else 0)
    check(lib().rs_sgd_step(layout, _ptr(p), _ptr(g), _ptr(buf), byref(hp), _ptr(tensor_mask),
                            _ptr(found_inf), k0, k1, _stream(stream)))


def rs_status_str(status: int) -> str:
    return lib().rs_status_str(status).decode()


def rs_last_error() -> str:
    return lib().rs_last_error().decode()


def ptr_table(tensors, device=None):
    """Device int64 array of the tensors' data pointers: the persistent
    tensor -> buffer mapping that rs_pack / rs_unpack read."""
    import torch
    ptrs = [t.data_ptr() for t in tensors]
    if device is None and not ptrs:
        raise ValueError("ptr_table: no tensors and no device")
    dev = device if device is not None else tensors[0].device
    return torch.tensor(ptrs, dtype=torch.int64, device=dev)


class Layout:
    """A planned, uploaded layout: owns the C handle, the device table and
    the sqnorm workspace (torch device allocations)."""

    def __init__(self, specs, m: int, S: int, offsets: Sequence[int], chunk_elems: int = 0,
                 device="cuda", stream=None):
        import torch
        self.specs = list(specs)
        self.m, self.S, self.offsets = m, S, list(offsets)
        self.handle = rs_layout_create(self.specs, m, S, self.offsets, chunk_elems)
        try:
            self.info = rs_layout_get_info(self.handle)
            self.table = torch.empty(self.info["device_bytes"], dtype=torch.uint8, device=device)
            rs_layout_upload(self.handle, self.table, stream)
            self.ws = torch.zeros(max(self.info["workspace_bytes"], 8), dtype=torch.uint8,
                                  device=device)
        except BaseException:
            self.close()  # the host tables are freed; the torch buffers go with self
            raise

    @classmethod
    def plan(cls, specs, m: int, align: int = 16, chunk_elems: int = 0, device="cuda",
             order=None):
        """Plan and build.  With `order` ("given", "block", "shape", "best")
        the tensors are laid out in that order: the layout's tensor i is
        specs[perm[i]], and `perm` is kept on the returned object."""
        specs = list(specs)
        if order is None:
            offs, info = rs_plan(specs, m, align)
            perm = list(range(len(specs)))
        else:
            perm, offs_by_t, info = rs_plan_ordered(specs, m, align, order)
            specs = [specs[t] for t in perm]
            offs = [offs_by_t[t] for t in perm]
        lay = cls(specs, m, info["S"], offs, chunk_elems, device)
        lay.plan_info = info
        lay.perm = perm
        return lay

    @property
    def total(self) -> int:
        return self.m * self.S

    @property
    def n(self) -> int:
        return len(self.specs)

    def close(self):
        if getattr(self, "handle", None) is not None:
            rs_layout_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
