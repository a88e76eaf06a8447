"""C-ABI checks that need no GPU: the library loads, exports every function
include/lsa.h declares, and the host-side validation and size queries behave
as documented (nothing reaches a kernel here)."""

import ctypes
import os
import re

import pytest

from sparse_attention_indexing_latent_amd import _lib
from sparse_attention_indexing_latent_amd._lib import CacheInfo, Layout, SelectCfg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "lsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", text)))


def _layout(**kw):
    base = dict(head_dim=128, latent_dim=64, n_kv_heads=8, n_q_heads=40, pool=4, block_entries=512,
                mean_bucket=8, max_bucket=16, dtype=_lib.LSA_BF16, build_tree=0)
    base.update(kw)
    return Layout(*[base[f] for f, _ in Layout._fields_])


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    decl = _declared()
    assert set(decl) == set(_lib.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name
    assert L.lsa_abi_version() == 7


def test_status_strings():
    L = _lib.lib()
    for code, name in _lib.STATUS_NAMES.items():
        assert L.lsa_status_string(code).decode() == name


@pytest.mark.parametrize("field,value,status", [
    ("latent_dim", 32, 2), ("pool", 2, 2), ("block_entries", 256, 2), ("mean_bucket", 4, 2),
    ("max_bucket", 32, 2), ("head_dim", 96, 2), ("n_q_heads", 41, 2), ("n_q_heads", 72, 2),
    ("dtype", 7, 3), ("build_tree", 2, 1), ("n_kv_heads", 0, 2),
])
def test_layout_validation(field, value, status):
    L = _lib.lib()
    lay = _layout(**{field: value})
    n = ctypes.c_size_t()
    assert L.lsa_cache_bytes(ctypes.byref(lay), 1, 4096, ctypes.byref(n)) == status
    assert L.lsa_last_error().decode()


def test_cache_bytes_and_describe():
    L = _lib.lib()
    lay = _layout(build_tree=1)
    n = ctypes.c_size_t()
    assert L.lsa_cache_bytes(ctypes.byref(lay), 2, 1 << 20, ctypes.byref(n)) == 0
    info = CacheInfo()
    assert L.lsa_cache_describe(ctypes.byref(lay), 2, 1 << 20, 1 << 20, ctypes.byref(info)) == 0
    assert info.n_blocks == 512 and info.n_leaves == 32768
    assert info.n_levels == 16 and info.level_size[15] == 1
    assert info.total_bytes == n.value
    # a smaller T inside the same cache
    assert L.lsa_cache_describe(ctypes.byref(lay), 2, 1 << 20, 5000, ctypes.byref(info)) == 0
    assert info.n_blocks == 2 and info.n_leaves == 128 and info.n_levels == 8
    # level offsets depend on the capacity only: level l has room for ceil(leaves_max / 2^l) nodes
    offs = [info.level_off[i] for i in range(1, info.n_levels)]
    room = [-(-info.leaves_max // (1 << i)) for i in range(1, info.n_levels)]
    assert all(offs[i + 1] == offs[i] + room[i] for i in range(len(offs) - 1))
    full = CacheInfo()
    assert L.lsa_cache_describe(ctypes.byref(lay), 2, 1 << 20, 1 << 20, ctypes.byref(full)) == 0
    assert all(full.level_off[i] == info.level_off[i] for i in range(1, info.n_levels))
    assert all(info.level_size[i] == -(-info.n_leaves // (1 << i)) for i in range(info.n_levels))
    assert L.lsa_cache_describe(ctypes.byref(lay), 2, 4096, 5000, ctypes.byref(info)) == 6


def test_extend_validation_before_launch():
    L = _lib.lib()
    lay = _layout(build_tree=1)
    fake = ctypes.c_void_p(0x1000)
    # T_new below T_old, beyond t_cap, beyond t_max
    assert L.lsa_extend_buckets(ctypes.byref(lay), fake, 1, 8192, 4096, 2048, fake, fake, 1 << 30, 8192, None) == 1
    assert L.lsa_extend_buckets(ctypes.byref(lay), fake, 1, 4096, 2048, 6144, fake, fake, 1 << 30, 8192, None) == 6
    assert L.lsa_extend_buckets(ctypes.byref(lay), fake, 1, 8192, 2048, 6144, fake, fake, 1 << 30, 4096, None) == 6
    # NULL / misaligned pointers, cache too small
    assert L.lsa_extend_buckets(ctypes.byref(lay), None, 1, 8192, 2048, 6144, fake, fake, 1 << 30, 8192, None) == 1
    assert L.lsa_extend_buckets(ctypes.byref(lay), ctypes.c_void_p(0x1001), 1, 8192, 2048, 6144, fake, fake,
                                1 << 30, 8192, None) == 4
    assert L.lsa_extend_buckets(ctypes.byref(lay), fake, 1, 8192, 2048, 6144, fake, fake, 16, 8192, None) == 5
    # nothing to do: no new full block
    assert L.lsa_extend_buckets(ctypes.byref(lay), fake, 1, 8192, 4096, 5000, fake, fake, 1 << 30, 8192, None) == 0


def test_build_validation_before_launch():
    L = _lib.lib()
    lay = _layout()
    fake = ctypes.c_void_p(0x1000)
    # T beyond t_cap / t_max
    assert L.lsa_build_buckets(ctypes.byref(lay), fake, 1, 100, 200, fake, fake, 1 << 30, 200, None) == 6
    assert L.lsa_build_buckets(ctypes.byref(lay), fake, 1, 300, 200, fake, fake, 1 << 30, 100, None) == 6
    # NULL / misaligned pointers
    assert L.lsa_build_buckets(ctypes.byref(lay), None, 1, 4096, 4096, fake, fake, 1 << 30, 4096, None) == 1
    assert L.lsa_build_buckets(ctypes.byref(lay), ctypes.c_void_p(0x1001), 1, 4096, 4096, fake, fake, 1 << 30,
                               4096, None) == 4
    # cache too small
    assert L.lsa_build_buckets(ctypes.byref(lay), fake, 1, 4096, 4096, fake, fake, 16, 4096, None) == 5


def test_select_validation_before_launch():
    L = _lib.lib()
    lay = _layout()
    fake = ctypes.c_void_p(0x1000)

    def call(cfg, lay=lay, ws=1 << 30, cache_bytes=1 << 30, T=8192, recs=None, rcnt=None):
        return L.lsa_select(ctypes.byref(lay), ctypes.byref(cfg), fake, cache_bytes, 8192, T, fake, fake, 1, 4,
                            fake, fake, fake, recs, rcnt, fake, ws, None)

    assert call(SelectCfg(2048, 4, 0, 0, 0, 0)) == 1             # window 0
    assert call(SelectCfg(-1, 4, 128, 0, 0, 0)) == 1             # negative k
    assert call(SelectCfg(5000, 4, 128, 0, 0, 0)) == 6           # k above LSA_MAX_K but below T
    assert call(SelectCfg(2048, 4, 128, 1, 0, 0)) == 6           # tree beam 0
    assert call(SelectCfg(2048, 4, 128, 1, 8, 0)) == 8           # tree on a cache without tree
    assert call(SelectCfg(2048, 4, 128, 0, 0, 9)) == 1           # unknown strategy
    assert call(SelectCfg(2048, 4, 128, 0, 0, 0, 2)) == 1        # causal_tree not 0 or 1
    assert call(SelectCfg(2048, 4, 128, 0, 0, 0, 0, 3)) == 1     # skip_recorded_lists not 0 or 1
    assert call(SelectCfg(2048, 4, 128, 0, 0, 0), ws=8) == 5     # workspace too small
    assert call(SelectCfg(2048, 4, 128, 0, 0, 0), T=9000) == 6   # T > t_max
    assert call(SelectCfg(2048, 4, 128, 0, 0, 0), cache_bytes=8) == 5
    assert call(SelectCfg(2048, 4, 128, 0, 0, 0), recs=fake) == 1                           # records without counts
    assert call(SelectCfg(2048, 4, 128, 0, 0, 0), recs=fake, rcnt=ctypes.c_void_p(0x1004)) == 4   # misaligned
    # k >= T is allowed even above LSA_MAX_K (every eligible token)
    n = ctypes.c_size_t()
    assert L.lsa_select_workspace_bytes(ctypes.byref(lay), ctypes.byref(SelectCfg(8192, 4, 128, 0, 0, 0)), 1, 4,
                                        8192, ctypes.byref(n)) == 0


def test_bucket_major_validation_before_launch():
    """Argument checks of lsa_sparse_attend_bucket_major, all before anything is launched."""
    L = _lib.lib()
    lay = _layout()
    cfg = SelectCfg(2048, 4, 1024, 0, 0, 0)
    fake = ctypes.c_void_p(0x1000)

    def call(recs=None, rcnt=None, lay=lay, ws=1 << 40, cache_bytes=1 << 40, fallback=None, batch=1):
        return L.lsa_sparse_attend_bucket_major(ctypes.byref(lay), ctypes.byref(cfg), fake, cache_bytes, 8192,
                                                fake, fake, fake, 8192, 8192, fake, batch, 4, fake, fake, recs, rcnt,
                                                ctypes.c_float(0.1), fake, fake, ws, fallback, None)

    assert call(recs=fake) == 1                                     # records without counts
    assert call(rcnt=fake) == 1                                     # counts without records
    assert call(recs=fake, rcnt=ctypes.c_void_p(0x1004)) == 4       # misaligned counts
    assert call(lay=_layout(dtype=_lib.LSA_F32)) == 8               # bf16 only
    assert call(cache_bytes=16) == 5                                # cache too small
    assert call(ws=16) == 5                                         # workspace too small
    assert call(fallback=ctypes.c_void_p(0x1008)) == 4              # misaligned fallback counters
    assert call(batch=1 << 21, cache_bytes=1 << 50) == 6                               # more (sequence, KV head) slices than a pass takes


def test_bucket_major_workspace_grows_per_query():
    """The workspace of a pass: fixed per-bin parts, plus per (query, KV head) a staging row of 256
    16-byte pair records and 80 pool slots (16 B of pair record, G rows of fp16 values and 16 B of
    max, denominator and scale)."""
    L = _lib.lib()
    lay = _layout()
    cfg = SelectCfg(2048, 4, 1024, 0, 0, 0)
    n1, n2 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.lsa_attend_bucket_major_workspace_bytes(ctypes.byref(lay), ctypes.byref(cfg), 1, 4096, 1 << 20,
                                                     ctypes.byref(n1)) == 0
    assert L.lsa_attend_bucket_major_workspace_bytes(ctypes.byref(lay), ctypes.byref(cfg), 1, 8192, 1 << 20,
                                                     ctypes.byref(n2)) == 0
    G, d = lay.n_q_heads // lay.n_kv_heads, lay.head_dim
    per_unit = 4 + 4 + 256 * 16 + 80 * (16 + G * (2 * d) + G * 16)
    units = 4096 * lay.n_kv_heads
    assert abs((n2.value - n1.value) - units * per_unit) <= 8 * 256 + 4 * units // 4096 * 2 + 16


def test_empty_calls_are_no_ops():
    L = _lib.lib()
    lay = _layout()
    cfg = SelectCfg(2048, 4, 1024, 0, 0, 0)
    # zero queries: nothing to do, no pointer is touched
    assert L.lsa_select(ctypes.byref(lay), ctypes.byref(cfg), None, 0, 0, 0, None, None, 1, 0, None, None, None,
                        None, None, None, 0, None) == 0
    assert L.lsa_sparse_attend(ctypes.byref(lay), ctypes.byref(cfg), None, None, None, 0, 0, None, 0, 5, None, None,
                               ctypes.c_float(0.1), None, None, 0, None) == 0


def test_attend_workspace_sizes():
    L = _lib.lib()
    lay = _layout()
    cfg = SelectCfg(2048, 4, 1024, 0, 0, 0)
    n = ctypes.c_size_t()
    # prefill-sized batches need no split workspace, decode-sized ones do
    assert L.lsa_attend_workspace_bytes(ctypes.byref(lay), ctypes.byref(cfg), 1, 65536, ctypes.byref(n)) == 0
    assert n.value == 0
    assert L.lsa_attend_workspace_bytes(ctypes.byref(lay), ctypes.byref(cfg), 16, 1, ctypes.byref(n)) == 0
    assert n.value > 0
