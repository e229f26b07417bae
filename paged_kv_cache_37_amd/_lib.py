"""ctypes view of libkvpool.so (include/kvpool.h).

torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process; streams and device memory are
shared with torch).  There is no fallback: without the built library the
import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading the library, see above)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvpool.so")

KVP_OK = 0
KVP_ERR_INVALID_ARG = -1
KVP_ERR_UNSUPPORTED = -2
KVP_ERR_WORKSPACE_TOO_SMALL = -3
KVP_ERR_HIP = -4

KVP_F32 = 0
KVP_BF16 = 1
KVP_FP8_E4M3 = 2

KVP_VARIANT_AUTO = 0
KVP_VARIANT_VALU = 1
KVP_VARIANT_MFMA = 2
KVP_VARIANT_STREAM = 3

NOALLOC_SCRATCH_BYTES = 64 << 20  # KVP_NOALLOC_SCRATCH_BYTES

EXPORTS = (
    "kv_pool_bytes",
    "kv_pool_create",
    "kv_pool_destroy",
    "kv_pool_describe",
    "kv_pool_set_fp8_scales",
    "kv_pool_offset",
    "cache_write",
    "paged_decode_workspace_bytes",
    "paged_decode_attention",
    "paged_decode_step",
    "paged_decode_step_noalloc",
    "kv_pool_copy_blocks",
    "paged_prefill_attention",
    "paged_prefill_step",
    "kvp_status_str",
    "kvp_last_error",
)


class PoolDesc(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("layer", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("sliding_window", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("partition_tokens", ctypes.c_int32),
        ("variant", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("shared_prefix_blocks", ctypes.c_int32),
        ("shared_blocks", ctypes.c_int32),
    ]


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("layer", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("cu_q_lens", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m paged_kv_cache_37_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    sig = {
        "kv_pool_bytes": (ctypes.c_size_t, [ctypes.POINTER(PoolDesc)]),
        "kv_pool_create": (i32, [ctypes.POINTER(PoolDesc), P, ctypes.c_size_t, ctypes.POINTER(P)]),
        "kv_pool_destroy": (i32, [P]),
        "kv_pool_describe": (i32, [P, ctypes.POINTER(PoolDesc)]),
        "kv_pool_set_fp8_scales": (i32, [P, i32, ctypes.c_float, ctypes.c_float]),
        "kv_pool_offset": (ctypes.c_int64, [P, i32, i32, i32, i32, i32, i32]),
        "cache_write": (i32, [P, i32, P, P, P, i32, P]),
        "paged_decode_workspace_bytes": (ctypes.c_size_t, [P, i32, i32, i32, i32]),
        "paged_decode_attention": (i32, [P, ctypes.POINTER(DecodeArgs), P]),
        "paged_decode_step": (i32, [P, ctypes.POINTER(DecodeArgs), P, P, P, P]),
        "paged_decode_step_noalloc": (i32, [P, ctypes.POINTER(DecodeArgs), P, P, P, P]),
        "kv_pool_copy_blocks": (i32, [P, P, P, i32, P]),
        "paged_prefill_attention": (i32, [P, ctypes.POINTER(PrefillArgs), P]),
        "paged_prefill_step": (i32, [P, ctypes.POINTER(PrefillArgs), P, P, P, P]),
        "kvp_status_str": (ctypes.c_char_p, [i32]),
        "kvp_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class KVPoolError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib.kvp_status_str(status).decode()
        detail = lib.kvp_last_error().decode()
        super().__init__(f"{what}: {msg}" + (f" ({detail})" if detail else ""))


def check(status: int, what: str) -> None:
    if status != KVP_OK:
        raise KVPoolError(status, what)
