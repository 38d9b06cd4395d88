"""Loader of libgrz.so (the HIP library) with its C signatures.

torch is imported first so that the HIP runtime torch ships is the one the
library binds to (both name it libamdhip64.so.7).  A missing library is an
error: there is no fallback of any kind.
"""

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime before libgrz)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgrz.so")

GRZ_OK, GRZ_EINVAL, GRZ_EINDIVISIBLE, GRZ_EALIGN, GRZ_EHIP, GRZ_ERANGE = range(6)
GRZ_F32, GRZ_BF16, GRZ_F64 = 0, 1, 2
(GRZ_SUM, GRZ_UNEVEN, GRZ_IN_COMPACT, GRZ_BF16_WIRE, GRZ_IN_RANGE, GRZ_ARGS_DEVICE,
 GRZ_OUT_GLOBAL, GRZ_IN_TILED, GRZ_MEAN_BF16, GRZ_COOPERATIVE) = (1, 2, 4, 8, 16, 32, 64, 128,
                                                                 256, 512)
GRZ_MAX_RANKS = 16
GRZ_PIECE = 4096
GRZ_NOALLOC_SCRATCH_BYTES = 65536

# Every symbol include/grz.h declares, with (restype, argtypes).
_vp, _i, _i64, _d = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
_pp = ctypes.POINTER(ctypes.c_void_p)


class Bucket(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("length", ctypes.c_int64)]


class AdamWArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float) for n in
                ("lr", "beta1", "beta2", "eps", "weight_decay", "bias_corr1", "bias_corr2")]


_BP = ctypes.POINTER(Bucket)
SIGNATURES = {
    "grz_version": (_i, []),
    "grz_strerror": (ctypes.c_char_p, [_i]),
    "grz_set_max_blocks": (_i, [_i]),
    "dp_ring_owned_chunk": (_i, [_i, _i]),
    "dp_ring_chunk_owner": (_i, [_i, _i]),
    "dp_chunk_range": (_i, [_i64, _i, _i, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "dp_piece_count": (_i64, [_BP, _i, _i, _i]),
    "dp_piece_offset": (_i64, [_BP, _i, _i, _i, _i, _i]),
    "dp_shard_numel": (_i64, [_BP, _i, _i, _i, _i]),
    "dp_tiled_numel": (_i64, [_BP, _i, _i, _i, _i]),
    "dp_reduce_scatter_mean": (_i, [_pp, _i, _i, _BP, _i, _i, _i, _vp, _vp, _vp]),
    "dp_reduce_scatter_mean_range": (_i, [_pp, _i, _i, _BP, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "dp_reduce_scatter_weighted": (_i, [_pp, ctypes.POINTER(_i64), _i, _i, _BP, _i, _i, _i, _i,
                                        _i, _vp, _vp, _vp]),
    "dp_grad_sqnorm_workspace": (ctypes.c_size_t, [_i64]),
    "dp_grad_sqnorm": (_i, [_vp, _i64, _d, _vp, _vp, _vp, _vp]),
    "dp_grad_sqnorm_noalloc": (_i, [_vp, _i64, _d, _vp, _vp, _vp]),
    "dp_grad_sqnorm_step_args": (_i, [_vp, _i64, _d, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "dp_grad_sqnorm_of_workspace": (ctypes.c_size_t, [_i64]),
    "dp_grad_sqnorm_of": (_i, [_vp, _i64, _d, _vp, _vp, _vp, _vp]),
    "zero1_adamw_step": (_i, [_vp, _vp, _vp, _vp, _i64, _vp, ctypes.POINTER(AdamWArgs), _vp,
                              _vp]),
    "zero1_adamw_gather": (_i, [_vp, _vp, _vp, _vp, _BP, _i, _i, _i, _i, _vp,
                                ctypes.POINTER(AdamWArgs), _pp, _i, _vp]),
    "zero1_all_gather": (_i, [_pp, _i, _BP, _i, _i, _pp, _i, _vp]),
    "dp_all_gather": (_i, [_pp, _i, _i, _BP, _i, _i, _pp, _i, _vp]),
    "grz_step_args_next": (_i, [_vp, _i64, _vp, _vp, _vp]),
    "zero1_fused_workspace": (ctypes.c_size_t, [_i64]),
    "zero1_fused_capacity": (_i64, [_i, _i]),
    "zero1_fused_step": (_i, [_pp, _i, _i, _BP, _i, _i, _i, _vp, _vp, _vp,
                              ctypes.POINTER(AdamWArgs), _d, _pp, _i, _vp, _vp, _vp, _vp, _vp,
                              _vp]),
    "zero1_fused_step_args": (_i, [_pp, _i, _i, _BP, _i, _i, _i, _vp, _vp, _vp, _vp, _i64, _vp,
                                   _vp, _d, _pp, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m gradient_reduce_zero_amd.build` "
                "(there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class GrzError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().grz_strerror(status).decode()
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def check(fn, status):
    if status != GRZ_OK:
        raise GrzError(fn, status)
