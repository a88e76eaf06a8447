"""Parity of the whole HIP path with the oracle on the tiny fp32 layer:
T = 8192, 1 KV head, 4 query heads, d = 64, 32 topics, k = 256, 4 sinks,
window 128, flat search.  Every block, every query and every output row is
compared."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_indexing_latent_amd as lsa
from synth import get_config, layer_inputs, random_lr_lists
from tests.parity import (check_lr_wellformed, compare_ward, gpu_partitions, lr_row, MARGIN, tol_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run1():
    print("[cfg1] generating inputs", flush=True)
    cfg = get_config(1)
    inp = layer_inputs(cfg, seed=0)
    dev = torch.device("cuda:0")
    G = {k: inp[k].to(dev).contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    print("[cfg1] build_buckets", flush=True)
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q, build_tree=True)
    torch.cuda.synchronize()
    K = inp["K"][0, 0].double().numpy()
    W = inp["W"].double().numpy()
    ocache = O.build_head_cache(K, W, "f32", tree=True)
    return dict(cfg=cfg, inp=inp, G=G, cache=cache, ocache=ocache, K=K, W=W,
                V=inp["V"][0, 0].double().numpy(), Q=inp["Q"][0].double().numpy())


def test_cfg1_ward_partitions_bit_exact(run1):
    gp = gpu_partitions(run1["cache"], 0, 0)
    st = compare_ward(run1["ocache"]["entries"], run1["ocache"]["clusters"], gp)
    print("[cfg1] ward", {k: v for k, v in st.items() if k != "margins"}, flush=True)
    assert st["unexcused"] == 0
    assert st["exact"] >= st["blocks"] - 1


def test_cfg1_cache_contents(run1):
    cache, oc = run1["cache"], run1["ocache"]
    cent = cache.centroids()[0, 0].double().cpu().numpy()
    sums = cache.sums()[0, 0].double().cpu().numpy()
    meta = cache.meta()[0, 0].cpu().numpy()
    eleaf = cache.entry_leaf()[0, 0].cpu().numpy()
    assert np.allclose(np.linalg.norm(cent, axis=1), 1.0, atol=1e-6)
    sizes = meta & 0xFF
    assert sizes.min() >= 1 and sizes.max() <= 16
    assert sizes.reshape(-1, 64).sum(axis=1).tolist() == [512] * (len(sizes) // 64)
    gp = gpu_partitions(cache, 0, 0)
    for blk, leaves in enumerate(gp):
        for r, mem in enumerate(leaves):
            assert all(eleaf[blk, e] == r for e in mem)
    # centroids and sums against the oracle on blocks whose partition matches
    for blk, (ocl, gcl) in enumerate(zip(oc["clusters"], gp)):
        if [list(c) for c in ocl] != gcl:
            continue
        sl = slice(64 * blk, 64 * blk + 64)
        assert np.max(np.abs(cent[sl] - oc["cent"][sl])) <= 1e-6
        assert np.max(np.abs(sums[sl] - oc["sums"][sl])) <= 1e-5


@pytest.mark.parametrize("strategy", ["materialized", "fused"])
def test_cfg1_select_flat(run1, strategy):
    cfg, G, oc = run1["cfg"], run1["G"], run1["ocache"]
    lr, cnt = lsa.select(G["Q"], run1["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window,
                         strategy=strategy)
    torch.cuda.synchronize()
    lr = lr[0, :, 0].cpu().numpy()
    cnt = cnt[0, :, 0].cpu().numpy()
    Q, W = run1["Q"], run1["W"]
    exact = excused = 0
    bad = []
    for t in range(cfg.T):
        row = lr_row(lr[t], cnt[t])
        check_lr_wellformed(row, cfg.k, t, oc["n_blocks"], cfg.n_sinks, cfg.window, int(cnt[t]))
        assert np.all(lr[t][max(cnt[t], 0):] == -1)
        qh = O.query_latent(Q[t], W, "f32")
        ref, info = O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window)
        if np.array_equal(ref, row):
            exact += 1
            continue
        _, info = O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, with_margin=True)
        if info["margin"] < MARGIN:
            excused += 1
        else:
            bad.append((t, info["margin"]))
    print(f"[cfg1] select {strategy}: exact {exact} excused {excused} unexcused {len(bad)}", flush=True)
    assert not bad, bad[:5]
    assert excused <= cfg.T // 100


def test_cfg1_attention_on_synthetic_lists(run1):
    cfg, G = run1["cfg"], run1["G"]
    idx, cnt = random_lr_lists(cfg, G["q_pos"].cpu(), seed=5, fill=0.5)
    dev = G["Q"].device
    Ogpu = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], idx.to(dev), cnt.to(dev), cfg.T, cfg.k,
                             cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    Ogpu = Ogpu[0].double().cpu().numpy()
    nb = cfg.T // 2048
    scale = 1 / math.sqrt(cfg.d)
    err = 0.0
    for t in range(0, cfg.T, 3):
        row = lr_row(idx[0, t, 0].numpy(), int(cnt[0, t, 0]))
        ref = O.attend(run1["Q"][t], run1["K"], run1["V"], t, row, cfg.n_sinks, cfg.window, nb, scale)
        err = max(err, float(np.max(np.abs(ref - Ogpu[t]))))
    print(f"[cfg1] attend max abs err {err:.3e}", flush=True)
    assert err <= tol_for("f32")


def test_cfg1_end_to_end(run1):
    cfg, G, oc = run1["cfg"], run1["G"], run1["ocache"]
    lr, cnt = lsa.select(G["Q"], run1["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window)
    Ogpu = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    Ogpu = Ogpu[0].double().cpu().numpy()
    scale = 1 / math.sqrt(cfg.d)
    err, compared = 0.0, 0
    for t in range(0, cfg.T, 5):
        qh = O.query_latent(run1["Q"][t], run1["W"], "f32")
        ref_lr, _ = O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window)
        if not np.array_equal(ref_lr, lr_row(lr[0, t, 0].cpu().numpy(), int(cnt[0, t, 0]))):
            continue
        ref = O.attend(run1["Q"][t], run1["K"], run1["V"], t, ref_lr, cfg.n_sinks, cfg.window, oc["n_blocks"], scale)
        err = max(err, float(np.max(np.abs(ref - Ogpu[t]))))
        compared += 1
    print(f"[cfg1] end-to-end rows {compared} max abs err {err:.3e}", flush=True)
    assert compared > 0.95 * len(range(0, cfg.T, 5))
    assert err <= tol_for("f32")


def test_cfg1_full_budget_is_dense_causal(run1):
    cfg, G = run1["cfg"], run1["G"]
    k = cfg.T
    lr, cnt = lsa.select(G["Q"], run1["cache"], G["q_pos"], G["W"], k, cfg.n_sinks, cfg.window)
    Ogpu = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, cfg.T, k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    Q = torch.from_numpy(run1["Q"]).permute(1, 0, 2).unsqueeze(0)            # [1, H, T, d]
    K = torch.from_numpy(run1["K"]).unsqueeze(0).unsqueeze(0).expand(1, cfg.H_q, -1, -1)
    V = torch.from_numpy(run1["V"]).unsqueeze(0).unsqueeze(0).expand(1, cfg.H_q, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=1 / math.sqrt(cfg.d))
    ref = ref[0].permute(1, 0, 2).numpy()
    err = float(np.max(np.abs(ref - Ogpu[0].double().cpu().numpy())))
    print(f"[cfg1] dense-equivalence max abs err {err:.3e}", flush=True)
    assert err <= tol_for("f32")


def test_cfg1_tree_matches_oracle(run1):
    cfg, G, oc = run1["cfg"], run1["G"], run1["ocache"]
    beam = 8
    lr, cnt = lsa.select(G["Q"], run1["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window,
                         search="tree", beam=beam)
    torch.cuda.synchronize()
    lr = lr[0, :, 0].cpu().numpy()
    cnt = cnt[0, :, 0].cpu().numpy()
    exact = excused = 0
    bad = []
    for t in range(0, cfg.T, 3):
        qh = O.query_latent(run1["Q"][t], run1["W"], "f32")
        ref, info = O.select_tree(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, beam, with_margin=True)
        row = lr_row(lr[t], cnt[t])
        if np.array_equal(ref, row):
            exact += 1
        elif info["margin"] < MARGIN:
            excused += 1
        else:
            bad.append((t, info["margin"]))
    print(f"[cfg1] tree beam {beam}: exact {exact} excused {excused} unexcused {len(bad)}", flush=True)
    assert not bad, bad[:5]
