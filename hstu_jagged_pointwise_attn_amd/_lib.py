"""ctypes loader for libhstu.so and the mirror of ``hstu_problem_t``.

The library is built in-tree (``build.py``). There is no fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhstu.so")

HSTU_OK, HSTU_ERR_INVALID_ARG, HSTU_ERR_UNSUPPORTED, HSTU_ERR_WORKSPACE, HSTU_ERR_HIP = range(5)
HSTU_BF16, HSTU_F32 = 0, 1
HSTU_NORM_NONE, HSTU_NORM_LN, HSTU_NORM_GLN = 0, 1, 2
HSTU_OP_FWD, HSTU_OP_BWD, HSTU_OP_MFALCON = 0, 1, 2
HSTU_MASK_CAND_TIME_FILTER = 1
HSTU_COST_TOKENS, HSTU_COST_ATTENTION = 0, 1
(HSTU_KERNEL_SCHED, HSTU_KERNEL_ATTN_FWD, HSTU_KERNEL_NORM_FWD, HSTU_KERNEL_NORM_BWD, HSTU_KERNEL_ATTN_BWD_DQ,
 HSTU_KERNEL_AUX, HSTU_KERNEL_ATTN_BWD_DKDV, HSTU_KERNEL_STOCHASTIC_LENGTH, HSTU_KERNEL_GATHER,
 HSTU_KERNEL_BALANCE, HSTU_KERNEL_GEMM, HSTU_KERNEL_LAYER_EW, HSTU_KERNEL_PROJ_SILU) = range(13)
HSTU_DEV_BAD_OFFSETS, HSTU_DEV_BAD_SEGMENTS, HSTU_DEV_BAD_GROUP, HSTU_DEV_TOO_LONG = 1, 2, 4, 8
HSTU_DEV_BAD_TIMESTAMPS = 16

_STATUS_NAMES = {1: "HSTU_ERR_INVALID_ARG", 2: "HSTU_ERR_UNSUPPORTED", 3: "HSTU_ERR_WORKSPACE",
                 4: "HSTU_ERR_HIP"}

_vp = ctypes.c_void_p


class Problem(ctypes.Structure):
    """Mirror of hstu_problem_t (include/hstu.h)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("max_len", ctypes.c_int32), ("n_max", ctypes.c_int32),
        ("offsets", _vp), ("prefix_len", _vp), ("cand_len", _vp), ("timestamps", _vp),
        ("rab_p", _vp), ("rab_t", _vp),
        ("n_pos", ctypes.c_int32), ("n_tb", ctypes.c_int32),
        ("norm", ctypes.c_int32), ("eps", ctypes.c_float),
        ("token_group", _vp),
        ("n_groups", ctypes.c_int32), ("mask_flags", ctypes.c_int32),
        ("gamma", _vp), ("beta", _vp),
    ]


class LayerWeights(ctypes.Structure):
    """Mirror of hstu_layer_weights_t (include/hstu.h)."""
    _fields_ = [("d_model", ctypes.c_int32), ("W1", _vp), ("b1", _vp), ("W2", _vp), ("b2", _vp)]


class StackLayer(ctypes.Structure):
    """Mirror of hstu_stack_layer_t (include/hstu.h)."""
    _fields_ = [("w", LayerWeights), ("rab_p", _vp), ("rab_t", _vp), ("gamma", _vp), ("beta", _vp),
                ("K_cache", _vp), ("V_cache", _vp)]


class HSTUError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None

# Every symbol include/hstu.h declares, with its argument types.
SIGNATURES = {
    "hstu_version": ([], ctypes.c_char_p),
    "hstu_last_error": ([], ctypes.c_char_p),
    "hstu_workspace_size": ([ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "hstu_tile_shape": ([ctypes.POINTER(Problem), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                         ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    "hstu_attn_fwd": ([ctypes.POINTER(Problem)] + [_vp] * 9 + [ctypes.c_size_t, _vp], ctypes.c_int),
    "hstu_attn_fwd_static": ([ctypes.POINTER(Problem)] + [_vp] * 9, ctypes.c_int),
    "hstu_static_scratch_bytes": ([], ctypes.c_size_t),
    "hstu_attn_bwd": ([ctypes.POINTER(Problem)] + [_vp] * 17 + [ctypes.c_size_t, _vp], ctypes.c_int),
    "hstu_mfalcon_score": ([ctypes.POINTER(Problem), _vp, ctypes.c_int64, ctypes.c_int32] + [_vp] * 7
                           + [ctypes.c_int32] + [_vp] * 5 + [ctypes.c_size_t, _vp], ctypes.c_int),
    "hstu_schedule_export": ([ctypes.POINTER(Problem), ctypes.c_int32, _vp, ctypes.c_int64, ctypes.c_int32,
                              ctypes.c_int32, _vp, ctypes.c_size_t, _vp, _vp, _vp, ctypes.c_int64,
                              ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
    "hstu_get_device_status": ([_vp, _vp, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    "hstu_kernel_timing": ([ctypes.c_int32], ctypes.c_int),
    "hstu_set_inline_schedule": ([ctypes.c_int32], ctypes.c_int32),
    "hstu_set_tile_order": ([ctypes.c_int32], ctypes.c_int32),
    "hstu_set_fused_projection": ([ctypes.c_int32], ctypes.c_int32),
    "hstu_kernel_timing_read": ([ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
    "hstu_stochastic_length": ([_vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                                _vp, _vp, _vp], ctypes.c_int),
    "hstu_gather_rows": ([_vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp, _vp], ctypes.c_int),
    "hstu_balance_bins": ([_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp], ctypes.c_int),
    "hstu_layer_workspace_size": ([ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "hstu_layer_fwd": ([ctypes.POINTER(Problem), ctypes.POINTER(LayerWeights)] + [_vp] * 9
                       + [ctypes.c_size_t, _vp], ctypes.c_int),
    "hstu_layer_bwd": ([ctypes.POINTER(Problem), ctypes.POINTER(LayerWeights)] + [_vp] * 18
                       + [ctypes.c_size_t, _vp], ctypes.c_int),
    "hstu_stack_workspace_size": ([ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "hstu_stack_history": ([ctypes.POINTER(Problem), ctypes.c_int32, ctypes.POINTER(StackLayer), _vp, _vp, _vp,
                            ctypes.c_size_t, _vp], ctypes.c_int),
    "hstu_stack_score": ([ctypes.POINTER(Problem), ctypes.c_int32, ctypes.POINTER(StackLayer), _vp, ctypes.c_int64,
                          ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "hstu_stack_score_capture": ([ctypes.POINTER(Problem), ctypes.c_int32, ctypes.POINTER(StackLayer), _vp,
                                  ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_size_t,
                                  ctypes.POINTER(_vp)], ctypes.c_int),
    "hstu_graph_launch": ([_vp, _vp], ctypes.c_int),
    "hstu_graph_destroy": ([_vp], ctypes.c_int),
}


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libhstu.so is not built ({LIB_PATH}); run `python -m hstu_jagged_pointwise_attn_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = res
        _lib = l
    return _lib


def check(status):
    if status != HSTU_OK:
        raise HSTUError(status, lib().hstu_last_error().decode(errors="replace"))
