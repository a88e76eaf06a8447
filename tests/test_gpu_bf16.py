"""Parity of the bf16 HIP path with the oracle on a layer shaped like the
131k prefill (GQA 10/2 heads here, head_dim 128, k = 2048, 4 sinks, window
1024) at T = 32768, small enough for the oracle to cover every Ward block and
a few thousand sampled (query, KV head) selections."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_indexing_latent_amd as lsa
from synth import get_config, layer_inputs, random_lr_lists
from tests.parity import (check_lr_wellformed, compare_ward, gpu_partitions, lr_row, MARGIN, tol_for)

pytestmark = pytest.mark.gpu

T_SMALL = 32768


@pytest.fixture(scope="module")
def runb():
    print("[bf16] generating inputs", flush=True)
    cfg = get_config(2, T=T_SMALL, H_kv=2, H_q=10, n_topics=64)
    inp = layer_inputs(cfg, seed=1)
    dev = torch.device("cuda:0")
    G = {k: inp[k].to(dev).contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    print("[bf16] build_buckets", flush=True)
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q, build_tree=True)
    torch.cuda.synchronize()
    W = inp["W"].double().numpy()
    Ks = [inp["K"][0, g].double().numpy() for g in range(cfg.H_kv)]
    print("[bf16] oracle caches", flush=True)
    ocaches = [O.build_head_cache(Ks[g], W, "bf16", tree=True, processes=8) for g in range(cfg.H_kv)]
    return dict(cfg=cfg, inp=inp, G=G, cache=cache, ocaches=ocaches, W=W, Ks=Ks,
                Vs=[inp["V"][0, g].double().numpy() for g in range(cfg.H_kv)], Q=inp["Q"][0].double().numpy())


def _sample_units(cfg, n, seed):
    rng = np.random.default_rng(seed)
    ts = rng.integers(0, cfg.T, n)
    gs = rng.integers(0, cfg.H_kv, n)
    return list(zip(ts.tolist(), gs.tolist()))


def test_bf16_ward_partitions(runb):
    cfg = runb["cfg"]
    tot = dict(blocks=0, exact=0, excused=0, unexcused=0)
    for g in range(cfg.H_kv):
        gp = gpu_partitions(runb["cache"], 0, g)
        oc = runb["ocaches"][g]
        st = compare_ward(oc["entries"], oc["clusters"], gp)
        for k in tot:
            tot[k] += st[k]
    print("[bf16] ward", tot, flush=True)
    assert tot["unexcused"] == 0
    assert tot["exact"] >= 0.9 * tot["blocks"]


def test_bf16_centroids(runb):
    cfg = runb["cfg"]
    cent = runb["cache"].centroids()[0].float().cpu().numpy()
    assert np.allclose(np.linalg.norm(cent, axis=2), 1.0, atol=4e-3)
    for g in range(cfg.H_kv):
        oc = runb["ocaches"][g]
        gp = gpu_partitions(runb["cache"], 0, g)
        for blk, (ocl, gcl) in enumerate(zip(oc["clusters"], gp)):
            if [list(c) for c in ocl] != gcl:
                continue
            sl = slice(64 * blk, 64 * blk + 64)
            d = np.abs(cent[g, sl] - oc["cent"][sl])
            assert d.max() <= 4e-3
            assert (d > 0).mean() < 0.01


def test_bf16_fused_equals_materialized(runb):
    cfg, G = runb["cfg"], runb["G"]
    a = lsa.select(G["Q"], runb["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, strategy="fused")
    b = lsa.select(G["Q"], runb["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window,
                   strategy="materialized")
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1])
    assert torch.equal(a[0], b[0])


@pytest.mark.parametrize("strategy", ["fused", "materialized"])
def test_bf16_select_flat_sampled(runb, strategy):
    cfg, G = runb["cfg"], runb["G"]
    lr, cnt = lsa.select(G["Q"], runb["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window,
                         strategy=strategy)
    torch.cuda.synchronize()
    lr = lr[0].cpu().numpy()
    cnt = cnt[0].cpu().numpy()
    exact = excused = 0
    bad = []
    units = _sample_units(cfg, 1500, 3)
    for t, g in units:
        oc = runb["ocaches"][g]
        row = lr_row(lr[t, g], cnt[t, g])
        check_lr_wellformed(row, cfg.k, t, oc["n_blocks"], cfg.n_sinks, cfg.window, int(cnt[t, g]))
        qh = O.query_latent(runb["Q"][t, g * cfg.G:(g + 1) * cfg.G], runb["W"], "bf16")
        ref, _ = O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window)
        if np.array_equal(ref, row):
            exact += 1
            continue
        _, info = O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, with_margin=True)
        if info["margin"] < MARGIN:
            excused += 1
        else:
            bad.append((t, g, info["margin"]))
    print(f"[bf16] select {strategy}: exact {exact} excused {excused} unexcused {len(bad)}", flush=True)
    assert not bad, bad[:5]
    assert excused <= 0.05 * len(units)


def test_bf16_tree_sampled(runb):
    cfg, G = runb["cfg"], runb["G"]
    beam = 64
    lr, cnt = lsa.select(G["Q"], runb["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window,
                         search="tree", beam=beam)
    torch.cuda.synchronize()
    lr = lr[0].cpu().numpy()
    cnt = cnt[0].cpu().numpy()
    exact = excused = 0
    bad = []
    for t, g in _sample_units(cfg, 800, 4):
        oc = runb["ocaches"][g]
        qh = O.query_latent(runb["Q"][t, g * cfg.G:(g + 1) * cfg.G], runb["W"], "bf16")
        ref, info = O.select_tree(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, beam, with_margin=True)
        row = lr_row(lr[t, g], cnt[t, g])
        if np.array_equal(ref, row):
            exact += 1
        elif info["margin"] < MARGIN:
            excused += 1
        else:
            bad.append((t, g, info["margin"]))
    print(f"[bf16] tree: exact {exact} excused {excused} unexcused {len(bad)}", flush=True)
    assert not bad, bad[:5]


def test_bf16_tree_full_beam_equals_flat_on_gpu():
    # 64 leaves visible at most (queries in block 1): a beam of 64 keeps every visible leaf
    cfg = get_config(2, T=4096, H_kv=2, H_q=10, n_topics=16)
    inp = layer_inputs(cfg, seed=9)
    dev = torch.device("cuda:0")
    G = {k: inp[k].to(dev).contiguous() for k in ("K", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q, build_tree=True)
    for k in (1, 100, 1000):
        a = lsa.select(G["Q"], cache, G["q_pos"], G["W"], k, 4, 128, search="tree", beam=64)
        b = lsa.select(G["Q"], cache, G["q_pos"], G["W"], k, 4, 128)
        torch.cuda.synchronize()
        assert torch.equal(a[1], b[1]) and torch.equal(a[0], b[0])


def test_bf16_attention_synthetic_lists(runb):
    cfg, G = runb["cfg"], runb["G"]
    idx, cnt = random_lr_lists(cfg, G["q_pos"].cpu()[:, :], seed=7, fill=0.3)
    dev = G["Q"].device
    Ogpu = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], idx.to(dev), cnt.to(dev), cfg.T, cfg.k,
                             cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    Ogpu = Ogpu[0].double().cpu().numpy()
    scale = 1 / math.sqrt(cfg.d)
    nb = cfg.T // 2048
    err = 0.0
    for t, g in _sample_units(cfg, 600, 5):
        row = lr_row(idx[0, t, g].numpy(), int(cnt[0, t, g]))
        ref = O.attend(runb["Q"][t, g * cfg.G:(g + 1) * cfg.G], runb["Ks"][g], runb["Vs"][g], t, row, cfg.n_sinks,
                       cfg.window, nb, scale)
        err = max(err, float(np.max(np.abs(ref - Ogpu[t, g * cfg.G:(g + 1) * cfg.G]))))
    print(f"[bf16] attend max abs err {err:.3e}", flush=True)
    assert err <= tol_for("bf16")


def test_bf16_end_to_end(runb):
    cfg, G = runb["cfg"], runb["G"]
    lr, cnt = lsa.select(G["Q"], runb["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window)
    Ogpu = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    Ogpu = Ogpu[0].double().cpu().numpy()
    lr = lr[0].cpu().numpy()
    cnt = cnt[0].cpu().numpy()
    scale = 1 / math.sqrt(cfg.d)
    err, compared, units = 0.0, 0, _sample_units(cfg, 400, 6)
    for t, g in units:
        oc = runb["ocaches"][g]
        qg = runb["Q"][t, g * cfg.G:(g + 1) * cfg.G]
        ref_lr, _ = O.select_flat(O.query_latent(qg, runb["W"], "bf16"), oc, t, cfg.k, cfg.n_sinks, cfg.window)
        if not np.array_equal(ref_lr, lr_row(lr[t, g], cnt[t, g])):
            continue
        ref = O.attend(qg, runb["Ks"][g], runb["Vs"][g], t, ref_lr, cfg.n_sinks, cfg.window, oc["n_blocks"], scale)
        err = max(err, float(np.max(np.abs(ref - Ogpu[t, g * cfg.G:(g + 1) * cfg.G]))))
        compared += 1
    print(f"[bf16] end-to-end rows {compared}/{len(units)} max abs err {err:.3e}", flush=True)
    assert compared >= 0.9 * len(units)
    assert err <= tol_for("bf16")


def test_bf16_full_budget_is_dense_causal():
    cfg = get_config(2, T=8192, H_kv=2, H_q=10, n_topics=16)
    inp = layer_inputs(cfg, seed=2)
    dev = torch.device("cuda:0")
    G = {k: inp[k].to(dev).contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q)
    k = cfg.T
    lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], k, cfg.n_sinks, cfg.window)
    Ogpu = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, cfg.T, k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    Q = inp["Q"][0].double().permute(1, 0, 2).unsqueeze(0)                      # [1, H_q, T, d]
    K = inp["K"][0].double().repeat_interleave(cfg.G, dim=0).unsqueeze(0)      # [1, H_q, T, d]
    V = inp["V"][0].double().repeat_interleave(cfg.G, dim=0).unsqueeze(0)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=1 / math.sqrt(cfg.d))
    ref = ref[0].permute(1, 0, 2).numpy()
    err = float(np.max(np.abs(ref - Ogpu[0].double().cpu().numpy())))
    print(f"[bf16] dense-equivalence max abs err {err:.3e}", flush=True)
    assert err <= tol_for("bf16")
