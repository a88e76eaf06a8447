"""Latent Sparse Attention (LSA) layer hot path for AMD Instinct MI355X.

Thin Python binding over liblsa.so (include/lsa.h).  The three calls follow
the method's problem statement (zhichai.net explainer "卡片柜", ch.2-ch.4):

    cache = build_buckets(K, W_k)                   # key side
    lr_idx, lr_cnt = select(Q, cache, q_pos, ...)   # query side selection
    O = sparse_attend(Q, K, V, q_pos, lr_idx, lr_cnt, ...)

Tensors live on the GPU (torch is used for device memory and the current
stream only); every step runs in the library's HIP kernels.
"""

from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional

import torch

from . import _lib
from ._lib import (LsaError, Layout, SelectCfg, CacheInfo, LSA_BF16, LSA_F32, LSA_SEARCH_FLAT, LSA_SEARCH_TREE,
                   LSA_STRATEGY_AUTO, LSA_STRATEGY_FUSED, LSA_STRATEGY_MATERIALIZED)

__all__ = ["build_buckets", "select", "sparse_attend", "sparse_attend_noalloc", "sparse_attend_bucket_major",
           "LsaCache", "LsaError",
           "make_layout", "select_cfg", "library_path", "select_workspace_bytes", "attend_workspace_bytes",
           "attend_bucket_major_workspace_bytes", "pca_projection"]

_STRATEGIES = {"auto": LSA_STRATEGY_AUTO, "fused": LSA_STRATEGY_FUSED, "materialized": LSA_STRATEGY_MATERIALIZED}


def library_path() -> str:
    return _lib.LIB_PATH


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return LSA_BF16
    if dt == torch.float32:
        return LSA_F32
    raise LsaError(3, f"unsupported dtype {dt}")


def make_layout(head_dim: int, n_kv_heads: int, n_q_heads: int, dtype: torch.dtype, build_tree: bool = False) -> Layout:
    return Layout(head_dim, _lib.LATENT_DIM, n_kv_heads, n_q_heads, _lib.POOL, _lib.BLOCK_ENTRIES,
                  _lib.MEAN_BUCKET, _lib.MAX_BUCKET, _dtype_code(dtype), 1 if build_tree else 0)


def select_cfg(k: int, n_sinks: int, window: int, search: str = "flat", beam: int = 0,
               strategy: str = "auto", causal_tree: bool = False, skip_recorded_lists: bool = False) -> SelectCfg:
    return SelectCfg(k, n_sinks, window, LSA_SEARCH_TREE if search == "tree" else LSA_SEARCH_FLAT, beam,
                     _STRATEGIES[strategy], int(causal_tree), int(skip_recorded_lists))


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclasses.dataclass
class LsaCache:
    """A bucket cache: an opaque device buffer plus the shape it was built for."""

    buf: torch.Tensor          # uint8 device buffer
    layout: Layout
    batch: int
    t_max: int
    T: int                     # tokens bucketed

    def info(self) -> CacheInfo:
        info = CacheInfo()
        _lib.check(_lib.lib().lsa_cache_describe(ctypes.byref(self.layout), self.batch, self.t_max, self.T,
                                                 ctypes.byref(info)))
        return info

    # ---- read-only views of the regions (inspection and tests)
    def _region(self, off, stride, count, dtype, shape):
        ebytes = torch.empty(0, dtype=dtype).element_size()
        HB = self.batch * self.layout.n_kv_heads
        raw = self.buf[off: off + stride * HB].view(HB, stride)[:, : count * ebytes]
        return raw.contiguous().view(dtype).view(self.batch, self.layout.n_kv_heads, *shape)

    def centroids(self) -> torch.Tensor:
        """[B, H_kv, n_leaves, 64] leaf centroids (bf16 storage is tile-swizzled: undone here)."""
        i = self.info()
        if self.layout.dtype != LSA_BF16:
            return self._region(i.off_cent, i.stride_cent, i.n_leaves * 64, torch.float32, (i.n_leaves, 64))
        nt = i.n_leaves // 16
        raw = self._region(i.off_cent, i.stride_cent, i.n_leaves * 64, torch.bfloat16, (nt, 2, 4, 16, 8))
        # stored (tile, m, h, r, e) -> bucket 16 tile + r, dim 16 h + 8 m + e
        return raw.permute(0, 1, 2, 5, 4, 3, 6).reshape(self.batch, self.layout.n_kv_heads, i.n_leaves, 64)

    def sums(self) -> torch.Tensor:
        i = self.info()
        return self._region(i.off_sums, i.stride_sums, i.n_leaves * 64, torch.float32, (i.n_leaves, 64))

    def meta(self) -> torch.Tensor:
        i = self.info()
        return self._region(i.off_meta, i.stride_meta, i.n_leaves, torch.int32, (i.n_leaves,))

    def members(self) -> torch.Tensor:
        i = self.info()
        return self._region(i.off_members, i.stride_members, i.n_blocks * 512, torch.int16, (i.n_blocks, 512))

    def entry_leaf(self) -> torch.Tensor:
        i = self.info()
        return self._region(i.off_entry_leaf, i.stride_entry_leaf, i.n_blocks * 512, torch.uint8, (i.n_blocks, 512))

    def entry_pos(self) -> torch.Tensor:
        """[B, H_kv, n_blocks, 512] position of each entry inside its bucket's member list."""
        i = self.info()
        return self._region(i.off_entry_pos, i.stride_entry_pos, i.n_blocks * 512, torch.uint8, (i.n_blocks, 512))

    def edge_table(self) -> torch.Tensor:
        """[B, H_kv, n_blocks_max + 1, levels, 64] tree only: row (nb, l) = centroid of the level-l node
        straddling leaf 64 nb over its leaves below it (rows of levels with no such node are unused)."""
        i = self.info()
        dt = torch.bfloat16 if self.layout.dtype == LSA_BF16 else torch.float32
        rows = (i.n_blocks_max + 1) * i.edge_levels
        return self._region(i.off_edge_cent, i.stride_edge_cent, rows * 64, dt,
                            (i.n_blocks_max + 1, i.edge_levels, 64))

    def tree_level(self, lev: int):
        """(centroids, sums) of tree level lev (0 = leaves)."""
        if lev == 0:
            return self.centroids(), self.sums()
        i = self.info()
        n, off = i.level_size[lev], i.level_off[lev]
        dt = torch.bfloat16 if self.layout.dtype == LSA_BF16 else torch.float32
        c = self._region(i.off_tree_cent, i.stride_tree_cent, i.nodes_max * 64, dt, (i.nodes_max, 64))
        s = self._region(i.off_tree_sums, i.stride_tree_sums, i.nodes_max * 64, torch.float32, (i.nodes_max, 64))
        return c[:, :, off: off + n], s[:, :, off: off + n]


def build_buckets(K: torch.Tensor, W_k: torch.Tensor, T: Optional[int] = None, t_max: Optional[int] = None,
                  build_tree: bool = False, n_q_heads: Optional[int] = None, cache: Optional[torch.Tensor] = None):
    """Key side: latent, normalise, pool, Ward per 512-entry block -> LsaCache.

    K: [B, H_kv, t_cap, d] (bf16 or fp32, contiguous, on the GPU); W_k: [d, 64].
    """
    assert K.is_cuda and K.is_contiguous() and W_k.is_contiguous()
    B, H_kv, t_cap, d = K.shape
    T = t_cap if T is None else T
    t_max = T if t_max is None else t_max
    layout = make_layout(d, H_kv, n_q_heads or H_kv, K.dtype, build_tree)
    L = _lib.lib()
    nbytes = ctypes.c_size_t()
    _lib.check(L.lsa_cache_bytes(ctypes.byref(layout), B, t_max, ctypes.byref(nbytes)))
    if cache is None:
        cache = torch.empty(nbytes.value, dtype=torch.uint8, device=K.device)
    _lib.check(L.lsa_build_buckets(ctypes.byref(layout), _ptr(K), B, t_cap, T, _ptr(W_k), _ptr(cache),
                                   cache.numel(), t_max, _stream(K.device)))
    return LsaCache(cache, layout, B, t_max, T)


def extend_buckets(cache: LsaCache, K: torch.Tensor, W_k: torch.Tensor, T_new: int) -> LsaCache:
    """Cache growth: cluster the full blocks of tokens [cache.T, T_new) of K and append their buckets
    (and the tree's new right edge) in place; the cache then equals a build of the first T_new tokens.

    K: [B, H_kv, t_cap, d] as for build_buckets, T_new <= t_cap and <= cache.t_max."""
    assert K.is_cuda and K.is_contiguous() and W_k.is_contiguous()
    B, H_kv, t_cap, d = K.shape
    _lib.check(_lib.lib().lsa_extend_buckets(ctypes.byref(cache.layout), _ptr(K), B, t_cap, cache.T, T_new,
                                             _ptr(W_k), _ptr(cache.buf), cache.buf.numel(), cache.t_max,
                                             _stream(K.device)))
    cache.T = T_new
    return cache


def select_workspace_bytes(cache: LsaCache, cfg: SelectCfg, n_q: int, n_q_heads: int) -> int:
    layout = Layout.from_buffer_copy(cache.layout)
    layout.n_q_heads = n_q_heads
    n = ctypes.c_size_t()
    _lib.check(_lib.lib().lsa_select_workspace_bytes(ctypes.byref(layout), ctypes.byref(cfg), cache.batch, n_q,
                                                     cache.t_max, ctypes.byref(n)))
    return n.value


def select(Q: torch.Tensor, cache: LsaCache, q_pos: torch.Tensor, W_q: torch.Tensor, k: int, n_sinks: int,
           window: int, search: str = "flat", beam: int = 0, strategy: str = "auto",
           workspace: Optional[torch.Tensor] = None, out: Optional[tuple] = None, causal_tree: bool = False,
           bucket_records: bool = False, skip_recorded_lists: bool = False):
    """Query side: score buckets, pick the top ones, expand to k tokens.

    Q: [B, n_q, H_q, d]; q_pos: int64 [B, n_q] on the GPU.  Returns
    (lr_idx int32 [B, n_q, H_kv, k] ascending, -1 padded; lr_cnt int32 [B, n_q, H_kv]).
    causal_tree (tree search): nodes straddling a query's visible leaves are scored by their visible
    part, as a decode step on a cache grown to the query's position would score them.
    bucket_records: also return the selection as bucket records, (recs int32 [B, n_q, H_kv, 256, 4]:
    leaf id, key mask low and high words, 0; counts int32 [B, n_q, H_kv], -1 where none), as a third
    item; out may then hold four tensors.  skip_recorded_lists (with bucket_records): rows that get
    records have no token list written (only for sparse_attend_bucket_major with those records).
    """
    assert Q.is_cuda and Q.is_contiguous() and q_pos.dtype == torch.int64 and q_pos.is_contiguous()
    B, n_q, H_q, d = Q.shape
    layout = Layout.from_buffer_copy(cache.layout)
    layout.n_q_heads = H_q
    cfg = select_cfg(k, n_sinks, window, search, beam, strategy, causal_tree, skip_recorded_lists)
    L = _lib.lib()
    H_kv = layout.n_kv_heads
    if out is None:
        lr_idx = torch.empty(B, n_q, H_kv, k, dtype=torch.int32, device=Q.device)
        lr_cnt = torch.empty(B, n_q, H_kv, dtype=torch.int32, device=Q.device)
        recs = rcnt = None
        if bucket_records:
            recs = torch.empty(B, n_q, H_kv, _lib.BUCKET_RECS, 4, dtype=torch.int32, device=Q.device)
            rcnt = torch.empty(B, n_q, H_kv, dtype=torch.int32, device=Q.device)
    else:
        lr_idx, lr_cnt = out[0], out[1]
        recs, rcnt = (out[2], out[3]) if bucket_records else (None, None)
    n = ctypes.c_size_t()
    _lib.check(L.lsa_select_workspace_bytes(ctypes.byref(layout), ctypes.byref(cfg), B, n_q, cache.t_max,
                                            ctypes.byref(n)))
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(n.value, 256), dtype=torch.uint8, device=Q.device)
    _lib.check(L.lsa_select(ctypes.byref(layout), ctypes.byref(cfg), _ptr(cache.buf), cache.buf.numel(),
                            cache.t_max, cache.T, _ptr(Q), _ptr(q_pos), B, n_q, _ptr(W_q),
                            _ptr(lr_idx) if k > 0 else ctypes.c_void_p(0), _ptr(lr_cnt),
                            _ptr(recs) if bucket_records else ctypes.c_void_p(0),
                            _ptr(rcnt) if bucket_records else ctypes.c_void_p(0), _ptr(workspace),
                            workspace.numel(), _stream(Q.device)))
    if bucket_records:
        return lr_idx, lr_cnt, (recs, rcnt)
    return lr_idx, lr_cnt


def attend_workspace_bytes(Q: torch.Tensor, H_kv: int, k: int, window: int) -> int:
    """Bytes of the split-key workspace sparse_attend needs for Q [B, n_q, H_q, d] (0: none)."""
    B, n_q, H_q, d = Q.shape
    layout = make_layout(d, H_kv, H_q, Q.dtype)
    n = ctypes.c_size_t()
    _lib.check(_lib.lib().lsa_attend_workspace_bytes(ctypes.byref(layout), ctypes.byref(select_cfg(k, 0, window)),
                                                     B, n_q, ctypes.byref(n)))
    return n.value


def sparse_attend(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, q_pos: torch.Tensor, lr_idx: torch.Tensor,
                  lr_cnt: torch.Tensor, T: int, k: int, n_sinks: int, window: int, scale: Optional[float] = None,
                  O: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact attention over sinks + window + selected tokens -> O [B, n_q, H_q, d]."""
    assert Q.is_contiguous() and K.is_contiguous() and V.is_contiguous()
    B, n_q, H_q, d = Q.shape
    _, H_kv, t_cap, _ = K.shape
    layout = make_layout(d, H_kv, H_q, Q.dtype)
    cfg = select_cfg(k, n_sinks, window)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if O is None:
        O = torch.empty_like(Q)
    L = _lib.lib()
    n = ctypes.c_size_t()
    _lib.check(L.lsa_attend_workspace_bytes(ctypes.byref(layout), ctypes.byref(cfg), B, n_q, ctypes.byref(n)))
    if n.value > 0 and (workspace is None or workspace.numel() < n.value):
        workspace = torch.empty(n.value, dtype=torch.uint8, device=Q.device)
    _lib.check(L.lsa_sparse_attend(ctypes.byref(layout), ctypes.byref(cfg), _ptr(Q), _ptr(K), _ptr(V), t_cap, T,
                                   _ptr(q_pos), B, n_q, _ptr(lr_idx) if k > 0 else ctypes.c_void_p(0), _ptr(lr_cnt),
                                   ctypes.c_float(scale), _ptr(O), _ptr(workspace) if n.value > 0 else ctypes.c_void_p(0),
                                   workspace.numel() if (workspace is not None and n.value > 0) else 0,
                                   _stream(Q.device)))
    return O


def sparse_attend_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, q_pos: torch.Tensor,
                          lr_idx: torch.Tensor, lr_cnt: torch.Tensor, T: int, k: int, n_sinks: int, window: int,
                          scale: Optional[float] = None, O: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_attend with the library's own fixed device scratch instead of a workspace (the C call
    allocates nothing; pass O to keep this wrapper allocation-free too)."""
    assert Q.is_contiguous() and K.is_contiguous() and V.is_contiguous()
    B, n_q, H_q, d = Q.shape
    _, H_kv, t_cap, _ = K.shape
    layout = make_layout(d, H_kv, H_q, Q.dtype)
    cfg = select_cfg(k, n_sinks, window)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if O is None:
        O = torch.empty_like(Q)
    _lib.check(_lib.lib().lsa_sparse_attend_noalloc(ctypes.byref(layout), ctypes.byref(cfg), _ptr(Q), _ptr(K), _ptr(V),
                                                    t_cap, T, _ptr(q_pos), B, n_q,
                                                    _ptr(lr_idx) if k > 0 else ctypes.c_void_p(0), _ptr(lr_cnt),
                                                    ctypes.c_float(scale), _ptr(O), _stream(Q.device)))
    return O


def attend_bucket_major_workspace_bytes(cache: LsaCache, n_q_heads: int, head_dim: int, n_q_pass: int) -> int:
    """Workspace bytes of one bucket-major pass over n_q_pass queries per sequence."""
    layout = make_layout(head_dim, cache.layout.n_kv_heads, n_q_heads, torch.bfloat16,
                         bool(cache.layout.build_tree))
    n = ctypes.c_size_t()
    _lib.check(_lib.lib().lsa_attend_bucket_major_workspace_bytes(ctypes.byref(layout),
                                                                  ctypes.byref(select_cfg(0, 0, 1)), cache.batch,
                                                                  n_q_pass, cache.t_max, ctypes.byref(n)))
    return n.value


def sparse_attend_bucket_major(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, q_pos: torch.Tensor,
                               lr_idx: torch.Tensor, lr_cnt: torch.Tensor, cache: LsaCache, k: int, n_sinks: int,
                               window: int, scale: Optional[float] = None, O: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None, n_q_pass: int = 16384,
                               bucket_records: Optional[tuple] = None,
                               fallback_counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_attend computed bucket-major (bf16): same outputs, each bucket's K/V read once per pass.

    Without a workspace, one for passes of min(n_q, n_q_pass) queries is allocated.  bucket_records:
    the (recs, counts) select returned with these lists (pairs taken from them; same output).
    fallback_counts: optional int32 [2] device tensor the call adds to: rows gathered whole instead,
    and of those the rows whose pairs did not fit in the pass's pool.
    """
    assert Q.is_contiguous() and K.is_contiguous() and V.is_contiguous()
    B, n_q, H_q, d = Q.shape
    _, H_kv, t_cap, _ = K.shape
    # the cache's own layout (build_tree included): the call finds the cache's regions from it
    assert cache.layout.head_dim == d and cache.layout.n_kv_heads == H_kv
    layout = make_layout(d, H_kv, H_q, Q.dtype, bool(cache.layout.build_tree))
    cfg = select_cfg(k, n_sinks, window)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if O is None:
        O = torch.empty_like(Q)
    if workspace is None:
        nbytes = attend_bucket_major_workspace_bytes(cache, H_q, d, max(1, min(n_q, n_q_pass)))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    _lib.check(_lib.lib().lsa_sparse_attend_bucket_major(
        ctypes.byref(layout), ctypes.byref(cfg), _ptr(cache.buf), cache.buf.numel(), cache.t_max, _ptr(Q), _ptr(K),
        _ptr(V), t_cap, cache.T, _ptr(q_pos), B, n_q, _ptr(lr_idx) if k > 0 else ctypes.c_void_p(0), _ptr(lr_cnt),
        _ptr(bucket_records[0]) if bucket_records is not None else ctypes.c_void_p(0),
        _ptr(bucket_records[1]) if bucket_records is not None else ctypes.c_void_p(0),
        ctypes.c_float(scale), _ptr(O), _ptr(workspace), workspace.numel(), _ptr(fallback_counts),
        _stream(Q.device)))
    return O


def pca_projection(K: torch.Tensor, T: Optional[int] = None, with_eigvals: bool = False):
    """Training-free projection: W [d, 64] = the 64 leading principal directions of the keys
    K [B, H_kv, t_cap, d] (first T positions), in K's dtype; optionally also all eigenvalues (fp32)."""
    assert K.is_cuda and K.is_contiguous()
    B, H_kv, t_cap, d = K.shape
    T = t_cap if T is None else T
    layout = make_layout(d, H_kv, H_kv, K.dtype)
    L = _lib.lib()
    n = ctypes.c_size_t()
    _lib.check(L.lsa_pca_workspace_bytes(ctypes.byref(layout), ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=K.device)
    W = torch.empty(d, _lib.LATENT_DIM, dtype=K.dtype, device=K.device)
    ev = torch.empty(d, dtype=torch.float32, device=K.device) if with_eigvals else None
    _lib.check(L.lsa_pca_projection(ctypes.byref(layout), _ptr(K), B, t_cap, T, _ptr(W), _ptr(ev), _ptr(ws),
                                    ws.numel(), _stream(K.device)))
    return (W, ev) if with_eigvals else W

