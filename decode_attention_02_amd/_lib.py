"""ctypes declarations of libmfa's C ABI (include/mfa.h).

Loads the in-tree ``libmfa.so``. There is no fallback: if the library is
missing or fails to load, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmfa.so")

MFA_OK = 0
MFA_F32, MFA_BF16, MFA_FP8_E4M3 = 0, 1, 2
MFA_WEIGHTS_ROWMAJOR, MFA_WEIGHTS_PACKED = 0, 1
BLOCK_TOKENS = 64
MAX_QUERY_TOKENS = 16
STATIC_SCRATCH = 32 << 20
ABI_VERSION = 3
STATUS_NAMES = {0: "MFA_OK", 1: "MFA_ERR_NULL", 2: "MFA_ERR_SHAPE", 3: "MFA_ERR_DTYPE",
                4: "MFA_ERR_ALIGN", 5: "MFA_ERR_UNSUPPORTED", 6: "MFA_ERR_WORKSPACE",
                7: "MFA_ERR_HIP", 8: "MFA_ERR_TOO_LARGE"}


class KVCacheDesc(ctypes.Structure):
    """mirror of ``mfa_kv_cache``"""
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class StepArgs(ctypes.Structure):
    """mirror of ``mfa_step_args``"""
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("d", ctypes.c_int), ("dtype", ctypes.c_int),
        ("x", ctypes.c_void_p), ("w_qdown", ctypes.c_void_p), ("w_qup", ctypes.c_void_p),
        ("q_norm_w", ctypes.c_void_p),
        ("hidden", ctypes.c_int), ("q_rank", ctypes.c_int), ("weight_layout", ctypes.c_int),
        ("eps", ctypes.c_float),
        ("qproj_workspace", ctypes.c_void_p), ("qproj_workspace_bytes", ctypes.c_size_t),
        ("q", ctypes.c_void_p),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("kv_in_dtype", ctypes.c_int),
        ("pos", ctypes.c_void_p),
        ("cache", ctypes.POINTER(KVCacheDesc)),
        ("seq_lens", ctypes.c_void_p),
        ("max_seq_len", ctypes.c_int),
        ("sm_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int), ("chunk_tokens", ctypes.c_int),
        ("split_workspace", ctypes.c_void_p), ("split_workspace_bytes", ctypes.c_size_t),
        ("out", ctypes.c_void_p),
        ("out_dtype", ctypes.c_int),
        ("w_kv", ctypes.c_void_p),
    ]


_i, _f, _p, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_pdesc = ctypes.POINTER(KVCacheDesc)
_pi = ctypes.POINTER(ctypes.c_int)

# name -> (restype, argtypes); the exact list of symbols include/mfa.h declares
SIGNATURES = {
    "mfa_abi_version": (_i, []),
    "mfa_status_str": (ctypes.c_char_p, [_i]),
    "mfa_qproj_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "mfa_qproj": (_i, [_p, _p, _p, _p, _p, _p, _sz, _i, _i, _i, _i, _i, _f, _i, _i, _p]),
    "mfa_pack_weight": (_i, [_p, _p, _i, _i, _i, _p]),
    "mfa_kv_append": (_i, [_p, _p, _i, _p, _i, _i, _pdesc, _p]),
    "mfa_decode_plan": (_i, [_i, _i, _i, _i, _i, _pi, _pi]),
    "mfa_decode_plan_lens": (_i, [_i, _i, _i, _p, _i, _pi, _pi]),
    "mfa_decode_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "mfa_split_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "mfa_decode_attn": (_i, [_p, _i, _i, _i, _pdesc, _p, _i, _f, _i, _i, _p, _sz, _p, _i, _p]),
    "mfa_decode_attn_static": (_i, [_p, _i, _i, _i, _pdesc, _p, _i, _f, _i, _i, _p, _i, _p]),
    "mfa_decode_attn_multi": (_i, [_p, _i, _i, _i, _i, _pdesc, _p, _i, _f, _i, _i, _p, _sz, _p,
                                   _i, _p]),
    "mfa_decode_attn_q8": (_i, [_p, _i, _i, _i, _i, _pdesc, _p, _i, _f, _i, _i, _p, _sz, _p,
                                _i, _p]),
    "mfa_combine": (_i, [_p, _sz, _i, _i, _i, _i, _p, _i, _p]),
    "mfa_out_proj_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "mfa_out_proj": (_i, [_p, _p, _i, _i, _i, _i, _i, _p, _sz, _p, _p, _p, _p]),
    "mfa_decode_step": (_i, [ctypes.POINTER(StepArgs), _p]),
}

_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmfa.so (once) and declare its signatures. Raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"libmfa.so not found at {path}: build it first "
            "(python -m decode_attention_02_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.mfa_abi_version() != ABI_VERSION:
        raise RuntimeError("libmfa.so ABI version mismatch")
    _LIB = lib
    return lib


class MfaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _LIB
        text = lib.mfa_status_str(status).decode() if lib is not None else "?"
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != MFA_OK:
        raise MfaError(fn, status)
