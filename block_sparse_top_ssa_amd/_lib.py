"""ctypes view of libssa.so (the C ABI declared in include/ssa.h)."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssa.so")

SSA_F32 = 0
SSA_BF16 = 1

STATUS = {
    0: "SSA_OK", 1: "SSA_ERR_NULL", 2: "SSA_ERR_SHAPE", 3: "SSA_ERR_DTYPE",
    4: "SSA_ERR_UNSUPPORTED", 5: "SSA_ERR_DEVICE", 6: "SSA_ERR_LAUNCH",
}

# Every symbol include/ssa.h declares, with its ctypes prototype.
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_F = ctypes.c_float


class Dims(ctypes.Structure):
    _fields_ = [("B", _I32), ("H", _I32), ("L", _I32), ("D", _I32), ("block", _I32), ("dtype", _I32),
                ("Hkv", _I32)]


_DP = ctypes.POINTER(Dims)
PROTOTYPES = {
    "ssa_block_pool": (_I32, [_DP, _VP, _VP, _VP]),
    "ssa_block_topk": (_I32, [_DP, _VP, _VP, _I32, _VP, _VP, _VP]),
    "ssa_sparse_attn_fwd": (_I32, [_DP, _VP, _VP, _VP, _VP, _I32, _F, _VP, _VP, _VP]),
    "ssa_full_attn_fwd": (_I32, [_DP, _VP, _VP, _VP, _F, _VP, _VP, _VP]),
    "ssa_kv_frag_bytes": (_I32, [_DP, ctypes.POINTER(ctypes.c_int64)]),
    "ssa_kv_frag": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP]),
    "ssa_sparse_attn_fwd_frag": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _F, _VP, _VP, _VP]),
    "ssa_full_attn_fwd_frag": (_I32, [_DP, _VP, _VP, _VP, _VP, _F, _VP, _VP, _VP]),
    "ssa_sparse_attn_fwd_stats": (_I32, [_DP, _VP, _VP, _VP, _VP, _I32, _F, _VP, _VP, _VP, _VP, _VP]),
    "ssa_full_attn_fwd_stats": (_I32, [_DP, _VP, _VP, _VP, _F, _VP, _VP, _VP, _VP, _VP]),
    "ssa_align_stats": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "ssa_align_stats_hist": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "ssa_decode_append": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "ssa_decode_sparse_fwd": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP, _I32, _F, _VP, _VP, _VP, _VP]),
    "ssa_decode_sparse_fwd_noalloc": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP, _I32, _F, _VP, _VP, _VP, _VP]),
    "ssa_decode_full_fwd": (_I32, [_DP, _VP, _VP, _VP, _VP, _F, _VP, _VP, _VP]),
    "ssa_full_attn_bwd": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _F, _VP, _VP, _VP, _VP]),
    "ssa_sparse_attn_bwd": (_I32, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _F, _VP, _VP, _VP, _VP]),
    "ssa_align_loss": (_I32, [_DP, _VP, _VP, _F, _F, _VP, _VP, _VP, _VP]),
    "ssa_attn_stats": (_I32, [_DP, _VP, _VP, _VP, _VP, _I32, _F, _VP, _VP, _VP]),
    "ssa_status_str": (ctypes.c_char_p, [_I32]),
    "ssa_last_error": (ctypes.c_char_p, []),
    "ssa_abi_version": (_I32, []),
    "ssa_set_kernel_variant": (_I32, [_I32]),
}

_lib = None


class SSAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.msg = msg


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libssa.so is not built at {path}; run `python -m block_sparse_top_ssa_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


PROBE_PATH = os.path.join(_PKG, "libssa_probe.so")
# include/ssa_probe.h (peak microbenchmarks, a separate library)
PROBE_PROTOTYPES = {
    "ssa_probe_mfma_bf16": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _VP, _VP]),
    "ssa_probe_hbm_read": (ctypes.c_int, [_VP, ctypes.c_size_t, ctypes.c_int, _VP, _VP]),
}


def load_probe(path: str = PROBE_PATH) -> ctypes.CDLL:
    """Load libssa_probe.so (raises if it has not been built)."""
    if not os.path.exists(path):
        raise ImportError(f"libssa_probe.so is not built at {path}; run `python -m block_sparse_top_ssa_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in PROBE_PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def check(code: int) -> None:
    if code != 0:
        raise SSAError(code, load().ssa_last_error().decode(errors="replace"))
