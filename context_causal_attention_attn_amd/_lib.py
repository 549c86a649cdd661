"""ctypes view of the C ABI declared in include/cp_attn.h.

Loading fails loudly (ImportError) when libcpattn.so has not been built: there
is no fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcpattn.so")

ABI_VERSION = 4
MAX_Q_CHUNKS = 16
MAX_KV_CHUNKS = 64
KV_CHUNK_ALIGN = 128
MAX_DOC_BOUNDS = 256

LAYOUT_CONTIGUOUS = 0
LAYOUT_HEAD_TAIL = 1
LAYOUT_CHUNKED = 2
LAYOUTS = {"contiguous": LAYOUT_CONTIGUOUS, "head_tail": LAYOUT_HEAD_TAIL, "chunked": LAYOUT_CHUNKED}

DTYPE_BF16 = 0
DTYPE_FP32 = 1

STATUS = {
    0: "OK", -1: "ERR_NULL_PTR", -2: "ERR_BAD_SHAPE", -3: "ERR_BAD_LAYOUT",
    -4: "ERR_BAD_POSITIONS", -5: "ERR_UNSUPPORTED", -6: "ERR_WORKSPACE", -7: "ERR_HIP",
    -8: "ERR_ABI", -9: "ERR_ALIGNMENT", -10: "ERR_DIVISIBILITY", -11: "ERR_SCRATCH_LIMIT",
}
NOALLOC_MAX_ROWS = 1 << 21

_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_p64 = ctypes.POINTER(ctypes.c_int64)


class CpAttnDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", _i32), ("dtype", _i32),
        ("batch", _i32), ("hq", _i32), ("hkv", _i32), ("head_dim", _i32),
        ("sq_local", _i64), ("skv", _i64),
        ("n_q_chunks", _i32), ("q_chunk_pos", _p64),
        ("n_kv_chunks", _i32), ("kv_chunk_pos", _p64),
        ("layout", _i32), ("causal", _i32), ("softmax_scale", _f32),
        ("q_strides", _i64 * 3), ("kv_strides", _i64 * 3), ("o_strides", _i64 * 3),
        ("n_docs", _i32), ("doc_starts", _p64),
        ("attn_mask", ctypes.c_void_p), ("mask_strides", _i64 * 3), ("mask_additive", _i32),
        ("chunk_strides", _i64 * 3),
    ]


class CpAttnPlanStats(ctypes.Structure):
    _fields_ = [
        ("work_items", _i64), ("kv_tile_visits", _i64), ("masked_tile_visits", _i64),
        ("block_q_rows", _i32), ("block_kv_rows", _i32), ("heads_per_item", _i32),
    ]


# Every symbol include/cp_attn.h declares, with its ctypes signature.
SIGNATURES = {
    "cp_attn_abi_version": (_i32, []),
    "cp_attn_error_string": (ctypes.c_char_p, [_i32]),
    "cp_attn_share_positions": (_i32, [_i32, _i64, _i32, _i32, _p64, ctypes.POINTER(_i32), _p64]),
    "cp_attn_validate": (_i32, [ctypes.POINTER(CpAttnDesc)]),
    "cp_attn_share_pairs": (_i32, [ctypes.POINTER(CpAttnDesc), _p64]),
    "cp_attn_workspace_bytes": (_i32, [ctypes.POINTER(CpAttnDesc), _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "cp_attn_plan_stats_fwd": (_i32, [ctypes.POINTER(CpAttnDesc), ctypes.POINTER(CpAttnPlanStats)]),
    "cp_attn_fwd": (_i32, [ctypes.POINTER(CpAttnDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                           ctypes.c_void_p]),
    "cp_attn_bwd": (_i32, [ctypes.POINTER(CpAttnDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "cp_attn_bwd_timed": (_i32, [ctypes.POINTER(CpAttnDesc), ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_void_p), _i32]),
    "cp_attn_bwd_noalloc": (_i32, [ctypes.POINTER(CpAttnDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "cp_attn_ulysses_relayout": (_i32, [_i32, _i32, _i32, _i32, _i32, _i64, _i32, ctypes.c_void_p,
                                        ctypes.c_void_p, _p64, ctypes.c_void_p]),
}

ULYSSES_STEPS = {"seq_to_head_pack": 0, "seq_to_head_unpack": 1,
                 "head_to_seq_pack": 2, "head_to_seq_unpack": 3}

_lib = None


def load() -> ctypes.CDLL:
    """Load libcpattn.so once. torch is imported first so that the library
    binds to the HIP runtime torch already loaded (same SONAME)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (pins the process's HIP runtime before dlopen)
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m context_causal_attention_attn_amd.build). There is no fallback path.")
    from . import build as _build
    if not _build.is_current(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} was built from other sources than the ones on disk: rebuild it "
            "(python -m context_causal_attention_attn_amd.build).")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.cp_attn_abi_version() != ABI_VERSION:
        raise ImportError(f"libcpattn ABI {lib.cp_attn_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


class CpAttnError(ValueError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().cp_attn_error_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


def check(status: int, where: str) -> None:
    if status != 0:
        raise CpAttnError(status, where)
