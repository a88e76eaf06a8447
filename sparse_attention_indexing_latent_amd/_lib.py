"""ctypes view of liblsa.so (the C ABI declared in include/lsa.h).

Argument marshalling only: every step of the LSA path runs in the HIP
kernels behind these symbols.  Importing this module fails loudly when the
library has not been built.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblsa.so")

LSA_F32, LSA_BF16 = 0, 1
LSA_SEARCH_FLAT, LSA_SEARCH_TREE = 0, 1
LSA_STRATEGY_AUTO, LSA_STRATEGY_FUSED, LSA_STRATEGY_MATERIALIZED = 0, 1, 2

LATENT_DIM = 64
POOL = 4
BLOCK_ENTRIES = 512
BLOCK_TOKENS = 2048
MEAN_BUCKET = 8
MAX_BUCKET = 16
LEAVES_PER_BLOCK = 64
MAX_GROUP = 8
MAX_K = 4096
MAX_BEAM = 64
BUCKET_RECS = 256

STATUS_NAMES = {
    0: "LSA_OK", 1: "LSA_ERR_INVALID_ARG", 2: "LSA_ERR_SHAPE", 3: "LSA_ERR_DTYPE", 4: "LSA_ERR_ALIGN",
    5: "LSA_ERR_WORKSPACE", 6: "LSA_ERR_CAPACITY", 7: "LSA_ERR_HIP", 8: "LSA_ERR_UNSUPPORTED",
}

# every symbol include/lsa.h declares
EXPORTS = [
    "lsa_cache_bytes", "lsa_cache_describe", "lsa_build_buckets", "lsa_extend_buckets", "lsa_select_workspace_bytes",
    "lsa_select",
    "lsa_attend_workspace_bytes", "lsa_sparse_attend", "lsa_sparse_attend_noalloc",
    "lsa_attend_bucket_major_workspace_bytes",
    "lsa_sparse_attend_bucket_major", "lsa_pca_workspace_bytes", "lsa_pca_projection", "lsa_status_string",
    "lsa_last_error", "lsa_abi_version",
]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "head_dim", "latent_dim", "n_kv_heads", "n_q_heads", "pool", "block_entries", "mean_bucket",
        "max_bucket", "dtype", "build_tree")]


class SelectCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("k", "n_sinks", "window", "search", "beam", "strategy", "causal_tree",
                                              "skip_recorded_lists")]


class CacheInfo(ctypes.Structure):
    _fields_ = [
        ("n_blocks_max", ctypes.c_int64), ("leaves_max", ctypes.c_int64), ("nodes_max", ctypes.c_int64),
        ("n_blocks", ctypes.c_int64), ("n_leaves", ctypes.c_int64), ("n_levels", ctypes.c_int32),
        ("elt_bytes", ctypes.c_int32), ("level_off", ctypes.c_int64 * 40), ("level_size", ctypes.c_int64 * 40),
    ] + [(n, ctypes.c_size_t) for n in (
        "off_cent", "off_sums", "off_meta", "off_members", "off_entry_leaf", "off_tree_cent", "off_tree_sums",
        "stride_cent", "stride_sums", "stride_meta", "stride_members", "stride_entry_leaf", "stride_tree_cent",
        "stride_tree_sums", "total_bytes", "off_entry_pos", "stride_entry_pos", "off_edge_cent", "stride_edge_cent")
    ] + [("edge_levels", ctypes.c_int32)] + [(n, ctypes.c_size_t) for n in (
        "off_cent_i8", "stride_cent_i8", "off_cent_scale", "stride_cent_scale")]


class LsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if liblsa.so is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_indexing_latent_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.lsa_cache_bytes.argtypes = [P(Layout), i64, i64, P(sz)]
    L.lsa_cache_describe.argtypes = [P(Layout), i64, i64, i64, P(CacheInfo)]
    L.lsa_build_buckets.argtypes = [P(Layout), vp, i64, i64, i64, vp, vp, sz, i64, vp]
    L.lsa_extend_buckets.argtypes = [P(Layout), vp, i64, i64, i64, i64, vp, vp, sz, i64, vp]
    L.lsa_select_workspace_bytes.argtypes = [P(Layout), P(SelectCfg), i64, i64, i64, P(sz)]
    L.lsa_select.argtypes = [P(Layout), P(SelectCfg), vp, sz, i64, i64, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, sz,
                             vp]
    L.lsa_attend_workspace_bytes.argtypes = [P(Layout), P(SelectCfg), i64, i64, P(sz)]
    L.lsa_sparse_attend.argtypes = [P(Layout), P(SelectCfg), vp, vp, vp, i64, i64, vp, i64, i64, vp, vp,
                                    ctypes.c_float, vp, vp, sz, vp]
    L.lsa_sparse_attend_noalloc.argtypes = [P(Layout), P(SelectCfg), vp, vp, vp, i64, i64, vp, i64, i64, vp, vp,
                                            ctypes.c_float, vp, vp]
    L.lsa_attend_bucket_major_workspace_bytes.argtypes = [P(Layout), P(SelectCfg), i64, i64, i64, P(sz)]
    L.lsa_sparse_attend_bucket_major.argtypes = [P(Layout), P(SelectCfg), vp, sz, i64, vp, vp, vp, i64, i64, vp,
                                                 i64, i64, vp, vp, vp, vp, ctypes.c_float, vp, vp, sz, vp, vp]
    L.lsa_pca_workspace_bytes.argtypes = [P(Layout), P(sz)]
    L.lsa_pca_projection.argtypes = [P(Layout), vp, i64, i64, i64, vp, vp, vp, sz, vp]
    for name in ("lsa_cache_bytes", "lsa_cache_describe", "lsa_build_buckets", "lsa_extend_buckets",
                 "lsa_select_workspace_bytes",
                 "lsa_select", "lsa_attend_workspace_bytes", "lsa_sparse_attend", "lsa_sparse_attend_noalloc",
                 "lsa_attend_bucket_major_workspace_bytes", "lsa_sparse_attend_bucket_major",
                 "lsa_pca_workspace_bytes", "lsa_pca_projection"):
        getattr(L, name).restype = ctypes.c_int
    L.lsa_status_string.argtypes = [ctypes.c_int]
    L.lsa_status_string.restype = ctypes.c_char_p
    L.lsa_last_error.argtypes = []
    L.lsa_last_error.restype = ctypes.c_char_p
    L.lsa_abi_version.argtypes = []
    L.lsa_abi_version.restype = ctypes.c_int32
    _lib = L
    return L


def check(status: int) -> None:
    if status != 0:
        raise LsaError(status, lib().lsa_last_error().decode())
