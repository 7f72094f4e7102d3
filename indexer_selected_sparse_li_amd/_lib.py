"""ctypes view of the C ABI declared in include/lisfa.h."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblisfa.so")

LISFA_OK = 0
LISFA_ERR_NULL_ARG = -1
LISFA_ERR_BAD_SHAPE = -2
LISFA_ERR_BAD_DTYPE = -3
LISFA_ERR_WORKSPACE = -4
LISFA_ERR_HIP = -5
LISFA_ERR_UNSUPPORTED = -6

LISFA_BF16 = 0
LISFA_FP8_E4M3 = 1
LISFA_MXFP8 = 2
LISFA_FP8_TILE128 = 3

LISFA_OP_TOPK = 0
LISFA_OP_SPARSE_MLA = 1
LISFA_OP_FUSED = 2
LISFA_OP_TOPK_CANDIDATES = 3
LISFA_OP_SPARSE_MLA_PARTIAL = 4
LISFA_OP_LI_TOPK = 5

LISFA_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = (
    "li_score", "li_topk", "li_topk_plan", "topk_select", "sparse_mla_attn", "li_topk_sfa", "li_topk_sfa_noalloc",
    "topk_candidates", "topk_merge", "sparse_mla_attn_partial", "lse_combine",
    "lisfa_zigzag_share", "zigzag_restore", "indexer_q_quant", "indexer_k_store", "indexer_prolog",
    "lisfa_workspace_size", "lisfa_status_string", "lisfa_struct_size", "lisfa_abi_version",
)


class Cache(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("num_slots", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("row_stride_bytes", ctypes.c_int32),
        ("scale", ctypes.c_void_p),
        ("scale_group_tokens", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("bt_stride", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("seq_base_slot", ctypes.c_void_p),
    ]


class IndexerArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p),
        ("q_scale_per_head", ctypes.c_int32),
        ("w", ctypes.c_void_p),
        ("k_cache", Cache),
        ("row_seq", ctypes.c_void_p),
        ("row_pos", ctypes.c_void_p),
        ("R", ctypes.c_int32),
        ("H_I", ctypes.c_int32),
        ("D_I", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int32),
        ("max_visible", ctypes.c_int64),
    ]


class MlaArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("kv_cache", Cache),
        ("row_seq", ctypes.c_void_p),
        ("R", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("D_latent", ctypes.c_int32),
        ("D_rope", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (never builds; call the build step first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m indexer_selected_sparse_li_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.li_score.argtypes = [ctypes.POINTER(IndexerArgs), vp, i64, vp]
    lib.li_score.restype = ctypes.c_int
    lib.li_topk.argtypes = [ctypes.POINTER(IndexerArgs), i32, vp, vp, sz, vp]
    lib.li_topk.restype = ctypes.c_int
    lib.li_topk_plan.argtypes = [ctypes.POINTER(IndexerArgs), i32, i32]
    lib.li_topk_plan.restype = i32
    lib.topk_select.argtypes = [vp, i64, vp, i32, i32, vp, vp, sz, vp]
    lib.topk_select.restype = ctypes.c_int
    lib.sparse_mla_attn.argtypes = [ctypes.POINTER(MlaArgs), vp, i32, vp, vp, vp, sz, vp]
    lib.sparse_mla_attn.restype = ctypes.c_int
    lib.li_topk_sfa.argtypes = [ctypes.POINTER(IndexerArgs), ctypes.POINTER(MlaArgs), i32, vp, vp, vp,
                                vp, sz, vp]
    lib.li_topk_sfa.restype = ctypes.c_int
    lib.li_topk_sfa_noalloc.argtypes = [ctypes.POINTER(IndexerArgs), ctypes.POINTER(MlaArgs), i32, vp, vp, vp, vp]
    lib.li_topk_sfa_noalloc.restype = ctypes.c_int
    lib.topk_candidates.argtypes = [vp, i64, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.topk_candidates.restype = ctypes.c_int
    lib.topk_merge.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, vp, vp]
    lib.topk_merge.restype = ctypes.c_int
    lib.sparse_mla_attn_partial.argtypes = [ctypes.POINTER(MlaArgs), vp, i32, vp, vp, vp, vp, sz, vp]
    lib.sparse_mla_attn_partial.restype = ctypes.c_int
    lib.lse_combine.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.lse_combine.restype = ctypes.c_int
    lib.lisfa_zigzag_share.argtypes = [i64, i32, i32, ctypes.POINTER(ctypes.c_int64)]
    lib.lisfa_zigzag_share.restype = ctypes.c_int
    lib.zigzag_restore.argtypes = [vp, vp, i64, i32, i64, vp]
    lib.zigzag_restore.restype = ctypes.c_int
    lib.indexer_q_quant.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.indexer_q_quant.restype = ctypes.c_int
    lib.indexer_k_store.argtypes = [vp, i32, i32, vp, vp, ctypes.c_float, i32, vp, vp, ctypes.POINTER(Cache), vp]
    lib.indexer_k_store.restype = ctypes.c_int
    lib.indexer_prolog.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp, ctypes.c_float, i32, vp, vp,
                                   ctypes.POINTER(Cache), vp]
    lib.indexer_prolog.restype = ctypes.c_int
    lib.lisfa_workspace_size.argtypes = [i32, i32, i64, i32, i32, i32]
    lib.lisfa_workspace_size.restype = sz
    lib.lisfa_status_string.argtypes = [i32]
    lib.lisfa_status_string.restype = ctypes.c_char_p
    lib.lisfa_struct_size.argtypes = [i32]
    lib.lisfa_struct_size.restype = sz
    lib.lisfa_abi_version.argtypes = []
    lib.lisfa_abi_version.restype = i32
    for which, cls in enumerate((Cache, IndexerArgs, MlaArgs)):
        if lib.lisfa_struct_size(which) != ctypes.sizeof(cls):
            raise RuntimeError(f"ABI mismatch for {cls.__name__}: library "
                               f"{lib.lisfa_struct_size(which)} bytes, binding {ctypes.sizeof(cls)}")
    _lib = lib
    return lib
