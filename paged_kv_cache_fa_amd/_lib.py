"""ctypes declarations of the C ABI in include/fa.h and the library loader."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; PKFA_LIB names another build of the same ABI to load
# instead (the tests use it for an AddressSanitizer build of the host paths).
LIB_PATH = os.environ.get("PKFA_LIB") or os.path.join(HERE, "libpkfa.so")

FA_OK = 0
FA_ERR_INVALID = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_CAPACITY = -4
FA_ERR_HIP = -5
FA_ERR_CAPTURING = -6
FA_ERR_NOT_PLANNED = -7
STATUS_NAMES = {
    FA_OK: "OK", FA_ERR_INVALID: "INVALID", FA_ERR_UNSUPPORTED: "UNSUPPORTED",
    FA_ERR_WORKSPACE: "WORKSPACE", FA_ERR_CAPACITY: "CAPACITY", FA_ERR_HIP: "HIP",
    FA_ERR_CAPTURING: "CAPTURING", FA_ERR_NOT_PLANNED: "NOT_PLANNED",
}

FA_F16, FA_BF16, FA_F32, FA_E4M3 = 0, 1, 2, 3
FA_MODE_DECODE, FA_MODE_APPEND = 0, 1

# every symbol declared in include/fa.h
EXPORTED = [
    "fa_workspace_size", "fa_plan", "fa_plan_info", "fa_plan_tiles", "fa_plan_destroy",
    "fa_plan_ragged", "fa_block_sparse_pages", "fa_decode", "fa_decode_noalloc", "fa_decode_scaled",
    "fa_decode_ragged", "fa_append",
    "fa_append_ragged", "fa_pod", "fa_cascade", "fa_merge_state", "fa_merge_states", "fa_status_string",
    "fa_last_error", "fa_probe_stream_read",
]


class Geometry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "mode", "dtype", "max_batch", "max_qo_tokens", "num_qo_heads", "num_kv_heads",
        "head_dim", "page_size", "num_cu", "tiles_per_cu", "min_chunk_pages", "qo_tile",
        "max_tiles", "max_partials", "max_merge", "pieces_per_worker", "kv_dtype")] + [
            ("reserved", ctypes.c_int32 * 7)]


class PlanT(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint64 * 64)]


class PlanStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tiles", "num_merge", "num_slots", "chunk_pages", "batch", "num_rows", "causal",
        "uploaded", "num_workers")] + [("resolved", Geometry)]


_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.code = STATUS_NAMES.get(status, str(status))


def load(path: str = LIB_PATH):
    """Load libpkfa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_cache_fa_amd.build`"
                          " or __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                           ctypes.c_size_t)
    GP = ctypes.POINTER(Geometry)
    PP = ctypes.POINTER(PlanT)
    sigs = {
        "fa_workspace_size": [GP, ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "fa_plan": [PP, GP, P, P, I32, P, I32, P, SZ, P, SZ, P],
        "fa_plan_ragged": [PP, GP, P, I32, P, I32, P, SZ, P, SZ, P],
        "fa_block_sparse_pages": [P, P, I32, P, I32, I32, P, P, I64, P, P, ctypes.POINTER(I64)],
        "fa_decode_ragged": [PP, P, P, P, I64, I64, P, F32, F32, F32, P, P, P],
        "fa_append_ragged": [PP, P, P, P, P, I64, I64, P, F32, P, P, P],
        "fa_pod": [PP, P, P, P, P, P, P, P, PP, P, P, P, P, P, P, P, P, I64, I64, I64, F32, P],
        "fa_plan_info": [PP, ctypes.POINTER(PlanStats)],
        "fa_plan_tiles": [PP, ctypes.POINTER(P), ctypes.POINTER(I32), ctypes.POINTER(P),
                          ctypes.POINTER(I32), ctypes.POINTER(P), ctypes.POINTER(I32)],
        "fa_plan_destroy": [PP],
        "fa_decode": [PP, P, P, P, I64, I64, I64, P, P, P, F32, P, P, P],
        "fa_decode_noalloc": [GP, P, P, I32, P, P, P, I64, I64, I64, P, P, P, F32, P, P, P],
        "fa_decode_scaled": [PP, P, P, P, I64, I64, I64, P, P, P, F32, F32, F32, P, P, P],
        "fa_append": [PP, P, P, P, P, I64, I64, I64, P, P, P, F32, P, P, P],
        "fa_cascade": [PP, PP, P, P, P, I64, I64, I64, P, P, P, P, P, P, P, F32, P, P, P, P, P, P,
                       P, P, P],
        "fa_merge_state": [P, P, P, P, P, P, I64, I32, I32, I32, P],
        "fa_merge_states": [P, P, I64, I32, I32, I32, I32, P, P, P],
        "fa_probe_stream_read": [P, I64, P, I32, P],
        "fa_status_string": [I32],
        "fa_last_error": [],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("fa_status_string", "fa_last_error") else I32
    _lib = lib
    return lib


def check(status: int):
    if status != FA_OK:
        detail = _lib.fa_last_error().decode() if _lib is not None else ""
        raise FAError(status, detail)
