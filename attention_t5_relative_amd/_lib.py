"""ctypes view of libfat5attn's C ABI (include/fat5attn.h).

Structures mirror the header field by field.  The shared library is loaded
from this package directory; if it has not been built the import of this
module raises, so no caller can run without the HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfat5attn.so")

FA_OK = 0
FA_ERR_INVALID = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_HIP = -4

FA_KERNEL_FWD = 0
FA_KERNEL_BWD_DQ = 1
FA_KERNEL_BWD_DKV = 2
FA_KERNEL_RMSNORM_FWD = 3
FA_KERNEL_RMSNORM_BWD = 4
FA_KERNEL_CE_FWD = 5
FA_KERNEL_CE_BWD = 6
FA_KERNEL_BWD_DBIAS_SUM = 7
FA_KERNEL_BWD_FIRE = 8
FA_KERNEL_COUNT = 9

FA_BWD_NOALLOC_MAX_BYTES = 16 << 20
FA_MFMA_PROBE_LANES = 2048 * 256

FA_BIAS_NONE = 0
FA_BIAS_T5 = 1
FA_BIAS_ALIBI = 2
FA_BIAS_DENSE = 3
FA_BIAS_FIRE = 4
FA_FIRE_MAX_HIDDEN = 64

c_i32 = ctypes.c_int32
c_f32 = ctypes.c_float
c_ptr = ctypes.c_void_p


class FaBias(ctypes.Structure):
    _fields_ = [("mode", c_i32), ("num_buckets", c_i32), ("max_distance", c_i32),
                ("bidirectional", c_i32), ("table", c_ptr), ("slopes", c_ptr),
                ("dense", c_ptr), ("dense_batch", c_i32), ("fire_hidden", c_i32)]


class FaFwdParams(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("seqlen", c_i32), ("heads", c_i32), ("head_dim", c_i32),
                ("causal", c_i32), ("scale", c_f32), ("rope_base", c_f32), ("reserved", c_i32),
                ("q", c_ptr), ("k", c_ptr), ("v", c_ptr), ("o", c_ptr), ("lse", c_ptr),
                ("bias", FaBias)]


class FaBwdParams(ctypes.Structure):
    _fields_ = [("f", FaFwdParams), ("dout", c_ptr), ("dq", c_ptr), ("dk", c_ptr),
                ("dv", c_ptr), ("dtable", c_ptr), ("dlse", c_ptr)]


class FaVarlenFwdParams(ctypes.Structure):
    _fields_ = [("nseq", c_i32), ("total", c_i32), ("max_seqlen", c_i32), ("heads", c_i32),
                ("head_dim", c_i32), ("causal", c_i32), ("scale", c_f32), ("rope_base", c_f32),
                ("cu_seqlens", c_ptr), ("q", c_ptr), ("k", c_ptr), ("v", c_ptr), ("o", c_ptr),
                ("lse", c_ptr), ("bias", FaBias)]


class FaVarlenBwdParams(ctypes.Structure):
    _fields_ = [("f", FaVarlenFwdParams), ("dout", c_ptr), ("dq", c_ptr), ("dk", c_ptr),
                ("dv", c_ptr), ("dtable", c_ptr), ("dlse", c_ptr)]


class FaRmsnormFwdParams(ctypes.Structure):
    _fields_ = [("rows", c_i32), ("dim", c_i32), ("eps", c_f32), ("reserved", c_i32),
                ("x", c_ptr), ("w", c_ptr), ("y", c_ptr), ("rstd", c_ptr)]


class FaRmsnormBwdParams(ctypes.Structure):
    _fields_ = [("f", FaRmsnormFwdParams), ("dy", c_ptr), ("dx", c_ptr), ("dw", c_ptr)]


class FaCeFwdParams(ctypes.Structure):
    _fields_ = [("rows", c_i32), ("vocab", c_i32), ("z_loss", c_f32), ("ignore_index", c_i32),
                ("logits", c_ptr), ("labels", c_ptr), ("loss", c_ptr), ("lse", c_ptr)]


class FaCeBwdParams(ctypes.Structure):
    _fields_ = [("f", FaCeFwdParams), ("dloss", c_ptr), ("dlogits", c_ptr)]


# Every symbol the header declares, with its ctypes signature.
SIGNATURES = {
    "fa_check_fwd": (c_i32, [ctypes.POINTER(FaFwdParams)]),
    "fa_check_bwd": (c_i32, [ctypes.POINTER(FaBwdParams)]),
    "fa_check_varlen_fwd": (c_i32, [ctypes.POINTER(FaVarlenFwdParams)]),
    "fa_check_varlen_bwd": (c_i32, [ctypes.POINTER(FaVarlenBwdParams)]),
    "fa_fwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(FaFwdParams)]),
    "fa_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(FaBwdParams)]),
    "fa_varlen_fwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(FaVarlenFwdParams)]),
    "fa_varlen_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(FaVarlenBwdParams)]),
    "fa_fwd": (c_i32, [ctypes.POINTER(FaFwdParams), c_ptr, ctypes.c_size_t, c_ptr]),
    "fa_bwd": (c_i32, [ctypes.POINTER(FaBwdParams), c_ptr, ctypes.c_size_t, c_ptr]),
    "fa_bwd_noalloc": (c_i32, [ctypes.POINTER(FaBwdParams), c_ptr]),
    "fa_varlen_fwd": (c_i32, [ctypes.POINTER(FaVarlenFwdParams), c_ptr, ctypes.c_size_t, c_ptr]),
    "fa_varlen_bwd": (c_i32, [ctypes.POINTER(FaVarlenBwdParams), c_ptr, ctypes.c_size_t, c_ptr]),
    "fa_t5_buckets": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_ptr, c_ptr]),
    "fa_rmsnorm_fwd": (c_i32, [ctypes.POINTER(FaRmsnormFwdParams), c_ptr]),
    "fa_rmsnorm_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(FaRmsnormBwdParams)]),
    "fa_rmsnorm_bwd": (c_i32, [ctypes.POINTER(FaRmsnormBwdParams), c_ptr, ctypes.c_size_t,
                               c_ptr]),
    "fa_ce_fwd": (c_i32, [ctypes.POINTER(FaCeFwdParams), c_ptr]),
    "fa_ce_bwd": (c_i32, [ctypes.POINTER(FaCeBwdParams), c_ptr]),
    "fa_set_kernel_timer": (c_i32, [c_i32, c_ptr, c_ptr]),
    "fa_mfma_probe": (c_i32, [c_i32, c_ptr, ctypes.POINTER(ctypes.c_double), c_ptr]),
    "fa_status_str": (ctypes.c_char_p, [c_i32]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_version": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libfat5attn.so from the package directory (raises if missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m attention_t5_relative_amd.build` "
            "(the attention path has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        self.status = status
        msg = lib.fa_status_str(status).decode()
        detail = lib.fa_last_error().decode()
        super().__init__(f"{where}: {msg} ({status}): {detail}")


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)
