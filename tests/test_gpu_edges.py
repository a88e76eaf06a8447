"""Edge cases of the HIP path against the oracle: ragged and tiny T, no
bucketed block, k = 0, no sinks, window 1 and window > T, several sequences
with decode positions, invalid positions, head_dim 64 in bf16, group sizes 1
and 8, odd tree shapes, and exact score ties (duplicated blocks) that the
lowest-id rule must break identically."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_indexing_latent_amd as lsa
from synth import get_config, layer_inputs
from tests.parity import MARGIN, check_lr_wellformed, lr_row, tol_for

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run_and_compare(cfg, inp, T_build, k, n_sinks, window, search="flat", beam=0, strategy="auto",
                     tree=False, positions=None, exact_only=False, check_attn=True):
    G = {kk: inp[kk].to(DEV).contiguous() for kk in ("K", "V", "W", "Q", "q_pos")}
    t_cap = G["K"].shape[2]
    cache = lsa.build_buckets(G["K"], G["W"], T=T_build, n_q_heads=cfg.H_q, build_tree=tree)
    lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], k, n_sinks, window, search=search, beam=beam,
                         strategy=strategy)
    Og = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, T_build, k, n_sinks, window)
    torch.cuda.synchronize()
    lr, cnt, Og = lr.cpu().numpy(), cnt.cpu().numpy(), Og.double().cpu().numpy()
    W = inp["W"].double().numpy()
    scale = 1 / math.sqrt(cfg.d)
    mism = 0
    err = 0.0
    for b in range(cfg.B):
        caches = [O.build_head_cache(inp["K"][b, g].double().numpy(), W, cfg.dtype, T=T_build, tree=tree)
                  for g in range(cfg.H_kv)]
        qp = inp["q_pos"][b].numpy()
        idxs = range(len(qp)) if positions is None else positions
        for i in idxs:
            t = int(qp[i])
            for g in range(cfg.H_kv):
                oc = caches[g]
                qg = inp["Q"][b, i, g * cfg.G:(g + 1) * cfg.G].double().numpy()
                qh = O.query_latent(qg, W, cfg.dtype)
                if search == "tree":
                    ref, info = O.select_tree(qh, oc, t, k, n_sinks, window, beam, with_margin=True)
                else:
                    ref, info = O.select_flat(qh, oc, t, k, n_sinks, window, with_margin=True)
                row = lr_row(lr[b, i, g], cnt[b, i, g]) if k > 0 else np.zeros(0, np.int64)
                check_lr_wellformed(row, k, t, oc["n_blocks"], n_sinks, window, int(cnt[b, i, g]),
                                    flat=search != "tree")
                if not np.array_equal(ref, row):
                    mism += 1
                    assert not exact_only, (b, i, g)
                    assert info["margin"] < MARGIN, (b, i, g, info["margin"])
                    continue
                if check_attn:
                    ref_o = O.attend(qg, inp["K"][b, g].double().numpy(), inp["V"][b, g].double().numpy(), t, ref,
                                     n_sinks, window, oc["n_blocks"], scale)
                    err = max(err, float(np.max(np.abs(ref_o - Og[b, i, g * cfg.G:(g + 1) * cfg.G]))))
    assert err <= tol_for(cfg.dtype), err
    return mism, err


def _cfg(**kw):
    base = dict(T=8192, H_kv=1, H_q=4, d=64, dtype="f32", n_topics=16, k=256, n_sinks=4, window=128)
    base.update(kw)
    return get_config(1, **base)


def test_ragged_T():
    cfg = _cfg(T=2048 * 3 + 777)
    inp = layer_inputs(cfg, seed=21)
    _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window, positions=range(0, cfg.T, 7))


def test_no_full_block_and_single_token():
    for T in (1, 5, 2047):
        cfg = _cfg(T=T)
        inp = layer_inputs(cfg, seed=22)
        _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window)


def test_zero_budget_no_sinks_window_one():
    cfg = _cfg(T=6144)
    inp = layer_inputs(cfg, seed=23)
    _run_and_compare(cfg, inp, cfg.T, 0, 4, 128, positions=range(0, cfg.T, 11))
    _run_and_compare(cfg, inp, cfg.T, 256, 0, 1, positions=range(0, cfg.T, 11))


def test_window_beyond_T():
    cfg = _cfg(T=6144)
    inp = layer_inputs(cfg, seed=24)
    _run_and_compare(cfg, inp, cfg.T, 256, 4, 100000, positions=range(0, cfg.T, 13))


def test_batch_of_decode_positions():
    cfg = _cfg(T=8192, B=3, H_kv=2, H_q=4)
    inp = layer_inputs(cfg, seed=25, T_cap=cfg.T + 1, q_positions=torch.full((3, 2), cfg.T, dtype=torch.int64))
    _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window, strategy="fused")


def test_invalid_position_gives_minus_one_and_zero_output():
    cfg = _cfg(T=4096)
    qp = torch.tensor([[-1, 100, 3000]], dtype=torch.int64)
    inp = layer_inputs(cfg, seed=26, q_positions=qp)
    G = {kk: inp[kk].to(DEV).contiguous() for kk in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q)
    for strategy in ("fused", "materialized"):
        lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, strategy=strategy)
        O_ = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
        torch.cuda.synchronize()
        assert int(cnt[0, 0, 0]) == -1 and bool((lr[0, 0, 0] == -1).all())
        assert bool((O_[0, 0] == 0).all())
        assert int(cnt[0, 1, 0]) == 0


@pytest.mark.parametrize("d,H_kv,H_q", [(64, 2, 4), (128, 4, 4), (128, 1, 8)])
def test_bf16_shapes(d, H_kv, H_q):
    cfg = get_config(2, T=8192, H_kv=H_kv, H_q=H_q, d=d, n_topics=16, k=512, window=256)
    inp = layer_inputs(cfg, seed=27)
    for strategy in ("fused", "materialized"):
        _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window, strategy=strategy,
                         positions=range(0, cfg.T, 17))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_materialized_tile_bound(dtype):
    # T = 32768: 64 tiles of 16 buckets per query against a first bound of max(16, k / 16) = 16
    # tiles, so the tile maxima decide which tiles' scores the finish reads
    cfg = _cfg(T=32768, dtype=dtype, d=128 if dtype == "bf16" else 64)
    inp = layer_inputs(cfg, seed=31, q_positions=torch.arange(20000, 32768, 397).unsqueeze(0))
    _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window, strategy="materialized")


def test_materialized_bound_widens_past_ineligible_tiles():
    # the keys of the last 4 blocks (inside the query's 8192-token window, so not eligible) all
    # repeat head 0's query: their 16 tiles score highest and hold no eligible token, so the
    # finish must widen its tile bound past them
    cfg = _cfg(T=32768, window=8192)
    t = cfg.T - 1
    inp = layer_inputs(cfg, seed=32, q_positions=torch.tensor([[t]]))
    inp["K"][0, 0, 24576:32768] = inp["Q"][0, 0, 0]
    _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window, strategy="materialized")


def test_materialized_exact_path_when_every_score_is_near_minus_one():
    # every key points against the (shared) query direction, so every bucket scores within 2^-11 of
    # -1: all sit in the finish's lowest histogram bin and the workgroup runs the exact radix path
    cfg = _cfg(T=8192)
    qp = torch.tensor([[3000, 5000, 8191]], dtype=torch.int64)
    inp = layer_inputs(cfg, seed=33, q_positions=qp)
    q0 = inp["Q"][0, 0, 0].clone()
    inp["Q"][0, :, :] = q0   # every head and query aims the same way
    g = torch.Generator().manual_seed(33)
    inp["K"][0, 0, :cfg.T] = -4.0 * q0 + 0.08 * torch.randn(cfg.T, cfg.d, generator=g)
    _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window, strategy="materialized")


def test_tree_odd_leaf_count():
    cfg = _cfg(T=2048 * 5)     # 320 leaves: levels 320, 160, 80, 40, 20, 10, 5, 3, 2, 1
    inp = layer_inputs(cfg, seed=28)
    for beam in (1, 3, 64):
        _run_and_compare(cfg, inp, cfg.T, cfg.k, cfg.n_sinks, cfg.window, search="tree", beam=beam, tree=True,
                         positions=range(0, cfg.T, 9))


def test_exact_ties_follow_lowest_id():
    # blocks 1 and 2 repeat block 0 exactly, so their buckets and centroids are
    # bit-identical and many scores tie exactly; the lowest bucket id must win
    cfg = _cfg(T=8192)
    inp = layer_inputs(cfg, seed=29)
    K = inp["K"]
    K[:, :, 2048:4096] = K[:, :, 0:2048]
    K[:, :, 4096:6144] = K[:, :, 0:2048]
    G = {kk: inp[kk].to(DEV).contiguous() for kk in ("K", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q)
    cent = cache.centroids()[0, 0]
    assert torch.equal(cent[0:64], cent[64:128]) and torch.equal(cent[0:64], cent[128:192])
    W = inp["W"].double().numpy()
    oc = O.build_head_cache(K[0, 0].double().numpy(), W, "f32")
    for strategy in ("fused", "materialized"):
        lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, strategy=strategy)
        torch.cuda.synchronize()
        lr, cnt = lr.cpu().numpy(), cnt.cpu().numpy()
        for t in range(6144, cfg.T, 3):
            qh = O.query_latent(inp["Q"][0, t].double().numpy(), W, "f32")
            ref, info = O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, with_margin=True)
            row = lr_row(lr[0, t, 0], cnt[0, t, 0])
            if np.array_equal(ref, row):
                continue
            # only a genuine near tie (the oracle's margin leaves exact duplicates to the id rule) may differ
            assert info["margin"] < MARGIN, (strategy, t, info["margin"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree_exact_ties_follow_lowest_id(dtype):
    # blocks 2..5 repeat blocks 0..1 exactly, so whole subtrees have bit-identical
    # centroids and the beam cut meets many exact ties at every level: the
    # lowest node index must win, as in the oracle
    kw = dict(T=12288) if dtype == "f32" else dict(T=12288, d=128, H_kv=1, H_q=4, n_topics=16, k=512, window=256)
    cfg = _cfg(**kw) if dtype == "f32" else get_config(2, **kw)
    inp = layer_inputs(cfg, seed=30)
    K = inp["K"]
    K[:, :, 4096:8192] = K[:, :, 0:4096]
    K[:, :, 8192:12288] = K[:, :, 0:4096]
    G = {kk: inp[kk].to(DEV).contiguous() for kk in ("K", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q, build_tree=True)
    W = inp["W"].double().numpy()
    oc = O.build_head_cache(K[0, 0].double().numpy(), W, cfg.dtype, tree=True)
    for beam in (64, 5):
        lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, search="tree",
                             beam=beam)
        torch.cuda.synchronize()
        lr, cnt = lr.cpu().numpy(), cnt.cpu().numpy()
        exact = 0
        for t in range(8192, cfg.T, 5):
            qh = O.query_latent(inp["Q"][0, t, : cfg.G].double().numpy(), W, cfg.dtype)
            ref, info = O.select_tree(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, beam, with_margin=True)
            row = lr_row(lr[0, t, 0], cnt[0, t, 0])
            if np.array_equal(ref, row):
                exact += 1
                continue
            # an exact tie (gap 0) must be broken as the oracle does: the oracle's margin (boundary gap
            # and level cuts, exact ties left to the index rule) must be a genuine near tie
            assert info["margin"] < MARGIN, (dtype, beam, t, info["margin"], info["cuts"])
        assert exact >= 0.9 * len(range(8192, cfg.T, 5)), (dtype, beam, exact)
