"""Cache growth (lsa_extend_buckets) and the causal tree search.

The pages cluster each block of 512 pooled keys once, as the keys stream in
(zhichai.net explainer, ch.2), and build the tree over the buckets (ch.4).
Growing a cache block by block must give, bit for bit, the cache a build of
the longer prefix gives; and a prefill query searching the tree in causal
mode must select exactly what a decode step at its position selects on the
cache grown to that point (the tree over the visible blocks only)."""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_indexing_latent_amd as lsa
from synth import get_config, layer_inputs
from tests.parity import MARGIN, check_lr_wellformed, lr_row

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _regions(cache, tree):
    out = {"cent": cache.centroids(), "sums": cache.sums(), "meta": cache.meta(), "members": cache.members(),
           "entry_leaf": cache.entry_leaf(), "entry_pos": cache.entry_pos()}
    if tree:
        i = cache.info()
        for lev in range(1, i.n_levels):
            c, s = cache.tree_level(lev)
            out[f"tcent{lev}"], out[f"tsums{lev}"] = c, s
        # edge rows in use: block boundaries 1..n_blocks, levels with a straddling node
        e = cache.edge_table()
        for nb in range(1, i.n_blocks + 1):
            for lev in range(1, i.n_levels):
                if (64 * nb) % (1 << lev):
                    out[f"edge{nb}_{lev}"] = e[:, :, nb, lev]
    return out


@pytest.mark.parametrize("dtype,tree,B", [("bf16", True, 1), ("f32", False, 1), ("f32", True, 2)])
def test_extend_equals_build(dtype, tree, B):
    if dtype == "bf16":
        cfg = get_config(2, T=2048 * 7 + 300, H_kv=2, H_q=10, d=128, n_topics=32, B=B)
    else:
        cfg = get_config(1, T=2048 * 7 + 300, H_kv=2, H_q=4, n_topics=32, B=B)
    inp = layer_inputs(cfg, seed=51, queries=False)
    K, W = inp["K"].to(DEV).contiguous(), inp["W"].to(DEV).contiguous()
    T = cfg.T
    a = lsa.build_buckets(K, W, T=T, t_max=T, build_tree=tree, n_q_heads=cfg.H_q)
    b = lsa.build_buckets(K, W, T=2 * 2048 + 5, t_max=T, build_tree=tree, n_q_heads=cfg.H_q)
    for T_new in (3 * 2048, 3 * 2048 + 100, T):   # one block, no new block, several blocks
        lsa.extend_buckets(b, K, W, T_new)
    torch.cuda.synchronize()
    ra, rb = _regions(a, tree), _regions(b, tree)
    assert ra.keys() == rb.keys()
    bad = [k for k in ra if not torch.equal(ra[k], rb[k])]
    assert not bad, bad


def test_extend_tree_levels_grow():
    """From 1 block (64 leaves, 7 levels) to 9 blocks (576 leaves, 11 levels): new levels appear."""
    cfg = get_config(1, T=2048 * 9, H_kv=1, H_q=4, n_topics=16)
    inp = layer_inputs(cfg, seed=52, queries=False)
    K, W = inp["K"].to(DEV).contiguous(), inp["W"].to(DEV).contiguous()
    a = lsa.build_buckets(K, W, T=cfg.T, build_tree=True, n_q_heads=cfg.H_q)
    b = lsa.build_buckets(K, W, T=2048, t_max=cfg.T, build_tree=True, n_q_heads=cfg.H_q)
    assert b.info().n_levels == 7
    for nb in range(2, 10):
        lsa.extend_buckets(b, K, W, 2048 * nb)
    torch.cuda.synchronize()
    assert b.info().n_levels == a.info().n_levels == 11
    ra, rb = _regions(a, True), _regions(b, True)
    bad = [k for k in ra if not torch.equal(ra[k], rb[k])]
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_tree_equals_decode_on_grown_cache(dtype):
    """Prefill queries with causal_tree on the whole cache select exactly what plain tree search selects on
    the cache built over the blocks each query can see (the cache a decode step at that position has)."""
    if dtype == "bf16":
        cfg = get_config(2, T=2048 * 11 + 77, H_kv=2, H_q=10, d=128, n_topics=32, k=512, window=256)
    else:
        cfg = get_config(1, T=2048 * 11 + 77, H_kv=2, H_q=4, n_topics=32)
    inp = layer_inputs(cfg, seed=53)
    G = {kk: inp[kk].to(DEV).contiguous() for kk in ("K", "W", "Q", "q_pos")}
    full = lsa.build_buckets(G["K"], G["W"], build_tree=True, n_q_heads=cfg.H_q)
    for beam in (2, 16):
        lr_c, cnt_c = lsa.select(G["Q"], full, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, search="tree",
                                 beam=beam, causal_tree=True)
        lr_p, cnt_p = lsa.select(G["Q"], full, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, search="tree",
                                 beam=beam)
        n_diff = 0
        for nvis in range(1, 12):
            lo, hi = 2048 * nvis, min(2048 * (nvis + 1), cfg.T)   # queries that see nvis blocks
            if lo >= hi:
                continue
            part = lsa.build_buckets(G["K"], G["W"], T=2048 * nvis, build_tree=True, n_q_heads=cfg.H_q)
            lr_d, cnt_d = lsa.select(G["Q"][:, lo:hi].contiguous(), part, G["q_pos"][:, lo:hi].contiguous(), G["W"],
                                     cfg.k, cfg.n_sinks, cfg.window, search="tree", beam=beam)
            torch.cuda.synchronize()
            assert torch.equal(cnt_c[:, lo:hi], cnt_d), (beam, nvis)
            assert torch.equal(lr_c[:, lo:hi], lr_d), (beam, nvis)
            n_diff += int((lr_c[:, lo:hi] != lr_p[:, lo:hi]).any(dim=-1).sum())
        print(f"[causal tree] {dtype} beam {beam}: {n_diff} (query, KV head) selections differ from the "
              f"stored-centroid search", flush=True)


def test_causal_tree_matches_oracle():
    cfg = get_config(1, T=2048 * 9 + 100, H_kv=1, H_q=4, n_topics=16)
    inp = layer_inputs(cfg, seed=54)
    G = {kk: inp[kk].to(DEV).contiguous() for kk in ("K", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], build_tree=True, n_q_heads=cfg.H_q)
    W = inp["W"].double().numpy()
    oc = O.build_head_cache(inp["K"][0, 0].double().numpy(), W, "f32", tree=True, processes=8)
    for beam in (3, 64):
        lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, search="tree",
                             beam=beam, causal_tree=True)
        torch.cuda.synchronize()
        lr, cnt = lr.cpu().numpy(), cnt.cpu().numpy()
        mism = 0
        for t in range(2048, cfg.T, 29):
            qh = O.query_latent(inp["Q"][0, t].double().numpy(), W, "f32")
            ref, info = O.select_tree(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, beam, with_margin=True, causal=True)
            row = lr_row(lr[0, t, 0], cnt[0, t, 0])
            check_lr_wellformed(row, cfg.k, t, oc["n_blocks"], cfg.n_sinks, cfg.window, int(cnt[0, t, 0]), flat=False)
            if not np.array_equal(ref, row):
                mism += 1
                assert info["margin"] < MARGIN, (beam, t, info["margin"])
        print(f"[causal tree] oracle parity beam {beam}: {mism} near-tie mismatches", flush=True)
