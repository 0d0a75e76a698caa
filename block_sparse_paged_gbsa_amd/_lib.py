"""ctypes binding of libgbsa.so (the C ABI declared in include/gbsa.h).

Argument marshalling only: every step of the computation runs in the HIP kernels of the
library. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgbsa.so")

METADATA_SIZE = 1024
HEAD_DIM = 128
PAGE_SIZE = 128
MAX_TOPK = 256
MAX_GROUP = 128
MAX_WORKERS = 999
MAX_BATCH = 16384

STATUS = {
    0: "GBSA_OK", 1: "GBSA_ERR_NULL", 2: "GBSA_ERR_SHAPE", 3: "GBSA_ERR_DTYPE",
    4: "GBSA_ERR_UNSUPPORTED", 5: "GBSA_ERR_EMPTY", 6: "GBSA_ERR_WORKSPACE",
    7: "GBSA_ERR_METADATA", 8: "GBSA_ERR_HIP",
}
DTYPE_F16, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
KV_PA_BBND, KV_TND = 0, 1
MAX_KV_ROWS = 2147483520

EXPORTED = ("gbsa_check_params", "gbsa_num_workers", "gbsa_metadata", "gbsa_workspace_size",
            "gbsa_forward", "gbsa_forward_tnd", "gbsa_forward_ex", "gbsa_forward_ex_noalloc",
            "gbsa_validate", "gbsa_status_string")
# the allocation-free forward's fixed device array (bytes) and counter limit (include/gbsa.h)
NOALLOC_SCRATCH_BYTES = 32 << 20
NOALLOC_MAX_COUNTERS = 16384
# gbsa_validate violation bits (include/gbsa.h)
VALIDATE_BITS = {0x01: "cu_seqlens_q", 0x02: "seqused_q", 0x04: "kv_length",
                 0x08: "cu_seqlens_kv", 0x10: "block_table", 0x20: "count", 0x40: "selection",
                 0x80: "mask_extent", 0x100: "max_seqlen"}
MASK_NONE, MASK_CAUSAL, MASK_CAUSAL_TOP_LEFT = 0, 1, 2


class GbsaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("total_q_blocks", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("block_x", ctypes.c_int32),
        ("block_y", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("kv_page_stride", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("mask_mode", ctypes.c_int32),
        ("win_left", ctypes.c_int32),
        ("win_right", ctypes.c_int32),
        ("quant_mode", ctypes.c_int32),
        ("softmax_precision", ctypes.c_int32),
        ("return_lse", ctypes.c_int32),
        ("is_packed_gqa", ctypes.c_int32),
        ("has_seqused_q", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("num_workers", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_kv", ctypes.c_int32),
        ("dst_type_max", ctypes.c_float),
    ]


class GbsaForwardArgs(ctypes.Structure):
    """gbsa_forward_args: every tensor of the main call (device pointers), the user mask's
    geometry, the workspace."""
    _fields_ = [
        ("query", ctypes.c_void_p),
        ("key", ctypes.c_void_p),
        ("value", ctypes.c_void_p),
        ("sparse_block_idx", ctypes.c_void_p),
        ("sparse_block_count", ctypes.c_void_p),
        ("metadata", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("seqused_q", ctypes.c_void_p),
        ("cu_seqlens_kv", ctypes.c_void_p),
        ("seqused_kv", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("p_scale", ctypes.c_void_p),
        ("atten_mask", ctypes.c_void_p),
        ("mask_batch_stride", ctypes.c_int64),
        ("mask_row_stride", ctypes.c_int64),
        ("mask_rows", ctypes.c_int32),
        ("mask_cols", ctypes.c_int32),
        ("attention_out", ctypes.c_void_p),
        ("softmax_lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class GbsaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}: {status_string(code)}")


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m block_sparse_paged_gbsa_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(GbsaParams)
    vp = ctypes.c_void_p
    lib.gbsa_check_params.argtypes = [P]
    lib.gbsa_check_params.restype = ctypes.c_int
    lib.gbsa_num_workers.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.gbsa_num_workers.restype = ctypes.c_int
    lib.gbsa_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.gbsa_workspace_size.restype = ctypes.c_int
    lib.gbsa_metadata.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.gbsa_metadata.restype = ctypes.c_int
    lib.gbsa_forward.argtypes = [P] + [vp] * 17 + [ctypes.c_size_t, vp]
    lib.gbsa_forward.restype = ctypes.c_int
    lib.gbsa_forward_tnd.argtypes = [P] + [vp] * 17 + [ctypes.c_size_t, vp]
    lib.gbsa_forward_tnd.restype = ctypes.c_int
    lib.gbsa_forward_ex.argtypes = [P, ctypes.POINTER(GbsaForwardArgs), vp]
    lib.gbsa_forward_ex.restype = ctypes.c_int
    lib.gbsa_forward_ex_noalloc.argtypes = [P, ctypes.POINTER(GbsaForwardArgs), vp]
    lib.gbsa_forward_ex_noalloc.restype = ctypes.c_int
    lib.gbsa_validate.argtypes = [P, ctypes.POINTER(GbsaForwardArgs), vp, vp]
    lib.gbsa_validate.restype = ctypes.c_int
    lib.gbsa_status_string.argtypes = [ctypes.c_int]
    lib.gbsa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().gbsa_status_string(int(code)).decode()


def check(fn: str, code: int) -> None:
    if code != 0:
        raise GbsaError(fn, code)
