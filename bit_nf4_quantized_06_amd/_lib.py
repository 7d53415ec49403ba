"""ctypes view of libqlora_nf4.so (the C ABI declared in include/qlora_nf4.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora_nf4.so")

QLORA_OK = 0
STATUS_NAMES = {0: "QLORA_OK", 1: "QLORA_ERR_NULL", 2: "QLORA_ERR_SHAPE", 3: "QLORA_ERR_ALIGN",
                4: "QLORA_ERR_WORKSPACE", 5: "QLORA_ERR_DEVICE", 6: "QLORA_ERR_HIP",
                7: "QLORA_ERR_FORMAT", 8: "QLORA_ERR_SCRATCH"}
FORMAT_VERSION = 1
BLOCKSIZE = 64
DQ_BLOCKSIZE = 256
QUANT_TYPES = {"nf4": 0, "int4": 1}          # QLORA_QUANT_*
COMPUTE_DTYPES = {"bf16": 0, "fp16": 1}      # QLORA_COMPUTE_*


class Nf4WeightDesc(ctypes.Structure):
    """Mirror of the C struct qlora_nf4_weight."""
    _fields_ = [
        ("format_version", ctypes.c_int32),
        ("blocksize", ctypes.c_int32),
        ("dq_blocksize", ctypes.c_int32),
        ("quant_type", ctypes.c_int16),
        ("compute_dtype", ctypes.c_int16),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("absmax_code", ctypes.c_void_p),
        ("absmax_scale", ctypes.c_void_p),
        ("absmax_offset", ctypes.c_void_p),
    ]


class DropoutDesc(ctypes.Structure):
    """Mirror of the C struct qlora_dropout."""
    _fields_ = [
        ("p", ctypes.c_double),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
    ]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_DESC_P = ctypes.POINTER(Nf4WeightDesc)
_DROP_P = ctypes.POINTER(DropoutDesc)

SIGNATURES = {
    "qlora_nf4_weight_init": (ctypes.c_int, [_DESC_P, _I64, _I64]),
    "qlora_nf4_weight_init_ex": (ctypes.c_int, [_DESC_P, _I64, _I64, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int]),
    "qlora_nf4_weight_buffer_sizes": (ctypes.c_int, [_DESC_P, ctypes.POINTER(_SZ),
                                                     ctypes.POINTER(_SZ), ctypes.POINTER(_SZ),
                                                     ctypes.POINTER(_SZ)]),
    "qlora_nf4_buffer_sizes": (ctypes.c_int, [_I64, _I64, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ),
                                              ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "qlora_nf4_quantize_workspace": (_SZ, [_I64, _I64]),
    "qlora_nf4_quantize": (ctypes.c_int, [_P, _DESC_P, _P, _SZ, _P]),
    "qlora_nf4_dequantize": (ctypes.c_int, [_DESC_P, _P, _P]),
    "qlora_nf4_merge": (ctypes.c_int, [_DESC_P, _P, _P, _I32, ctypes.c_float, _P, _P]),
    "qlora_adamw_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_double,
                                        ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_double, _P]),
    "qlora_adamw_step16": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_double, _P]),
    "qlora_linear_workspace": (_SZ, [_I64, _I64, _I64, _I32, ctypes.c_int]),
    "qlora_set_pre_dequant_min_tokens": (_I64, [_I64]),
    "qlora_pre_dequant_min_tokens": (_I64, []),
    "qlora_linear_fwd": (ctypes.c_int, [_DESC_P, _P, _I64, _P, _P, _I32, ctypes.c_float, _P, _P,
                                        _P, _SZ, _P]),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_DESC_P, _P, _I64, _P, _P, _I32, ctypes.c_float,
                                                _P, _P, _P]),
    "qlora_linear_fwd_noalloc_max_scratch": (_SZ, []),
    "qlora_linear_bwd": (ctypes.c_int, [_DESC_P, _P, _P, _I64, _P, _P, _I32, ctypes.c_float, _P,
                                        _P, _P, _P, _P, _SZ, _P]),
    "qlora_dropout_mask_bytes": (_SZ, [_I64, _I64]),
    "qlora_dropout_mask": (ctypes.c_int, [_DROP_P, _I64, _I64, _P, _P, _P, _P]),
    "qlora_linear_workspace_dropout": (_SZ, [_I64, _I64, _I64, _I32, ctypes.c_int]),
    "qlora_linear_fwd_dropout": (ctypes.c_int, [_DESC_P, _P, _I64, _P, _P, _I32, ctypes.c_float,
                                                _DROP_P, _P, _P, _P, _P, _P, _SZ, _P]),
    "qlora_linear_bwd_dropout": (ctypes.c_int, [_DESC_P, _P, _P, _I64, _P, _P, _I32,
                                                ctypes.c_float, _DROP_P, _P, _P, _P, _P, _P,
                                                _P, _P, _SZ, _P]),
    "qlora_set_timing_events": (ctypes.c_int, [ctypes.c_int, _P, _P]),
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_last_hip_error": (ctypes.c_int, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (after torch, whose HIP runtime it links)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  -- brings torch's libamdhip64 into the process first
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`"
                " (the HIP library is required; there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class QloraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        msg = lib.qlora_status_string(status).decode()
        extra = ""
        if status == 6:
            extra = f" (hipError_t {lib.qlora_last_hip_error()})"
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}{extra}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != QLORA_OK:
        raise QloraError(fn, status)
