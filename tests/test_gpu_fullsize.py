"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (65,536-query chunks, fused flat search; tree search at 10M).

* 131,072-token prefill (8 KV / 40 query heads): the oracle rebuilds the whole
  bucket cache from K (every Ward block) and recomputes sampled selections and
  outputs on its own.
* 1M prefill, 16 x 1M decode and 10M tree prefill: the oracle recomputes
  sampled Ward blocks from K; selections are checked against the oracle's
  selection rule applied to the cache the GPU built (the GPU's buckets and
  centroids as data), plus the properties every list has; attention is
  checked on synthetic index lists against the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_indexing_latent_amd as lsa
from synth import decode_inputs, get_config, layer_inputs, random_lr_lists
from tests.parity import (MARGIN, check_lr_wellformed, compare_ward, gpu_partitions, lr_row, tol_for,
                          ward_first_divergence_margin)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CHUNK = 65536


def _cache_dict_from_gpu(cache, b, g, tree=False):
    """The GPU-built cache of (b, g) as the oracle's cache structure."""
    meta = cache.meta()[b, g].cpu().numpy().astype(np.int64)
    mem = cache.members()[b, g].cpu().numpy().astype(np.int64) & 0xFFFF
    nb = mem.shape[0]
    members = []
    for x in range(len(meta)):
        blk = x // 64
        sz, off = meta[x] & 0xFF, (meta[x] >> 8) & 0x3FF
        members.append(mem[blk, off:off + sz] + 512 * blk)
    d = dict(n_blocks=nb, members=members, cent=cache.centroids()[b, g].double().cpu().numpy(),
             sums=cache.sums()[b, g].double().cpu().numpy())
    if tree:
        info = cache.info()
        levels = [dict(cent=d["cent"], span=1, first_leaf=np.arange(len(meta)))]
        for lev in range(1, info.n_levels):
            c, s = cache.tree_level(lev)
            levels.append(dict(cent=c[b, g].double().cpu().numpy(), sums=s[b, g].double().cpu().numpy(),
                               span=1 << lev, first_leaf=np.arange(0, len(meta), 1 << lev)))
        d["tree"] = levels
    return d


def _sampled_ward(inp_K, W, cache, pairs):
    """pairs of (b, g, block): oracle Ward from K vs the GPU partition."""
    stats = dict(blocks=0, exact=0, excused=0, unexcused=0)
    gp_cache = {}
    for (b, g, blk) in pairs:
        if (b, g) not in gp_cache:
            gp_cache[(b, g)] = gpu_partitions(cache, b, g)
        Kb = inp_K[b, g, blk * 2048:(blk + 1) * 2048].double().cpu().numpy()
        E = O.pooled_entries(O.key_latents(Kb, W))
        oc = O.ward_block(E)["clusters"]
        gc = gp_cache[(b, g)][blk]
        stats["blocks"] += 1
        if [list(c) for c in oc] == gc:
            stats["exact"] += 1
        elif ward_first_divergence_margin(E, gc) < MARGIN:
            stats["excused"] += 1
        else:
            stats["unexcused"] += 1
    return stats


def _check_selection(qh, gcache, t, row, cnt, cfg, tree, beam):
    """Oracle selection rule on the given cache; the margin (slow at 10M
    leaves) is computed only when the lists differ."""
    def run(with_margin):
        if tree:
            return O.select_tree(qh, gcache, t, cfg.k, cfg.n_sinks, cfg.window, beam, with_margin=with_margin)
        return O.select_flat(qh, gcache, t, cfg.k, cfg.n_sinks, cfg.window, with_margin=with_margin)
    check_lr_wellformed(row, cfg.k, t, gcache["n_blocks"], cfg.n_sinks, cfg.window, cnt, flat=not tree)
    ref, _ = run(False)
    if np.array_equal(ref, row):
        return "exact"
    _, info = run(True)
    return "excused" if info["margin"] < MARGIN else "unexcused"


def test_prefill_131k_full_oracle():
    cfg = get_config(2)
    print("[131k] generating", flush=True)
    inp = layer_inputs(cfg, seed=0, device=DEV)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q)
    lr = torch.empty(1, cfg.T, cfg.H_kv, cfg.k, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, cfg.T, cfg.H_kv, dtype=torch.int32, device=DEV)
    Og = torch.empty_like(G["Q"])
    for i0 in range(0, cfg.T, CHUNK):
        sl = slice(i0, i0 + CHUNK)
        lsa.select(G["Q"][:, sl], cache, G["q_pos"][:, sl], G["W"], cfg.k, cfg.n_sinks, cfg.window,
                   strategy="fused", out=(lr[:, sl], cnt[:, sl]))
        lsa.sparse_attend(G["Q"][:, sl], G["K"], G["V"], G["q_pos"][:, sl], lr[:, sl], cnt[:, sl], cfg.T, cfg.k,
                          cfg.n_sinks, cfg.window, O=Og[:, sl])
    torch.cuda.synchronize()
    W = G["W"].double().cpu().numpy()
    print("[131k] oracle caches (all 512 Ward blocks)", flush=True)
    ward = dict(blocks=0, exact=0, excused=0, unexcused=0)
    ocaches = []
    for g in range(cfg.H_kv):
        Kg = G["K"][0, g].double().cpu().numpy()
        oc = O.build_head_cache(Kg, W, "bf16", processes=12)
        st = compare_ward(oc["entries"], oc["clusters"], gpu_partitions(cache, 0, g))
        for k in ward:
            ward[k] += st[k]
        ocaches.append(oc)
    print("[131k] ward", ward, flush=True)
    assert ward["unexcused"] == 0 and ward["exact"] >= 0.95 * ward["blocks"]
    rng = np.random.default_rng(11)
    lr_c, cnt_c, O_c = lr[0].cpu().numpy(), cnt[0].cpu().numpy(), Og[0].float().cpu().numpy()
    KV = {}
    res = dict(exact=0, excused=0, unexcused=0)
    err = 0.0
    scale = 1 / math.sqrt(cfg.d)
    for _ in range(256):
        t, g = int(rng.integers(0, cfg.T)), int(rng.integers(0, cfg.H_kv))
        qg = G["Q"][0, t, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
        qh = O.query_latent(qg, W, "bf16")
        row = lr_row(lr_c[t, g], cnt_c[t, g])
        ref, info = O.select_flat(qh, ocaches[g], t, cfg.k, cfg.n_sinks, cfg.window, with_margin=True)
        check_lr_wellformed(row, cfg.k, t, ocaches[g]["n_blocks"], cfg.n_sinks, cfg.window, int(cnt_c[t, g]))
        if np.array_equal(ref, row):
            res["exact"] += 1
            if g not in KV:
                KV[g] = (G["K"][0, g].double().cpu().numpy(), G["V"][0, g].double().cpu().numpy())
            ref_o = O.attend(qg, KV[g][0], KV[g][1], t, ref, cfg.n_sinks, cfg.window, ocaches[g]["n_blocks"], scale)
            err = max(err, float(np.max(np.abs(ref_o - O_c[t, g * cfg.G:(g + 1) * cfg.G]))))
        else:
            res["excused" if info["margin"] < MARGIN else "unexcused"] += 1
    print(f"[131k] select {res} attend max abs err {err:.2e}", flush=True)
    assert res["unexcused"] == 0 and res["exact"] >= 240
    assert err <= tol_for("bf16")


def _sampled_fullsize(cfg, inp, cache, lr, cnt, units, tree=False, beam=0, q_of=None, t_of=None):
    """units: (b, i, g) triples; checks selection against the GPU cache data."""
    W = inp["W"].double().cpu().numpy()
    gcaches = {}
    res = dict(exact=0, excused=0, unexcused=0)
    for (b, i, g) in units:
        if (b, g) not in gcaches:
            gcaches[(b, g)] = _cache_dict_from_gpu(cache, b, g, tree)
        t = t_of(b, i)
        qg = q_of(b, i, g)
        qh = O.query_latent(qg, W, "bf16")
        row = lr_row(lr[b, i, g], int(cnt[b, i, g]))
        res[_check_selection(qh, gcaches[(b, g)], t, row, int(cnt[b, i, g]), cfg, tree, beam)] += 1
    return res


def test_prefill_1m_sampled():
    cfg = get_config(4)
    print("[1m] generating", flush=True)
    inp = layer_inputs(cfg, seed=0, device=DEV)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q)
    rng = np.random.default_rng(4)
    W = G["W"].double().cpu().numpy()
    pairs = [(0, int(rng.integers(0, cfg.H_kv)), int(rng.integers(0, cfg.T // 2048))) for _ in range(24)]
    ward = _sampled_ward(G["K"], W, cache, pairs)
    print("[1m] ward", ward, flush=True)
    assert ward["unexcused"] == 0 and ward["exact"] >= 22
    # two chunks as bench launches them: the first and one late in the sequence
    for i0 in (0, cfg.T - CHUNK):
        sl = slice(i0, i0 + CHUNK)
        lr, cnt = lsa.select(G["Q"][:, sl], cache, G["q_pos"][:, sl], G["W"], cfg.k, cfg.n_sinks, cfg.window,
                             strategy="fused")
        torch.cuda.synchronize()
        lr_c, cnt_c = lr.cpu().numpy(), cnt.cpu().numpy()
        units = [(0, int(rng.integers(0, CHUNK)), int(rng.integers(0, cfg.H_kv))) for _ in range(40)]
        res = _sampled_fullsize(cfg, G, cache, lr_c, cnt_c, units,
                                q_of=lambda b, i, g: G["Q"][b, i0 + i, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy(),
                                t_of=lambda b, i: i0 + i)
        print(f"[1m] chunk {i0} select {res}", flush=True)
        assert res["unexcused"] == 0 and res["exact"] >= 36
    # the late chunk as the prefill bench times it: bucket records, no lists for the rows that have them,
    # bucket-major passes of 32768 queries; equal to the same call on the lists, and to the gather call
    Qc, qpc = G["Q"][:, sl].contiguous(), G["q_pos"][:, sl].contiguous()
    lr_r = torch.empty_like(lr)
    cnt_r = torch.empty_like(cnt)
    recs = torch.empty(1, CHUNK, cfg.H_kv, 256, 4, dtype=torch.int32, device=DEV)
    rcnt = torch.empty(1, CHUNK, cfg.H_kv, dtype=torch.int32, device=DEV)
    lsa.select(Qc, cache, qpc, G["W"], cfg.k, cfg.n_sinks, cfg.window, strategy="fused", bucket_records=True,
               skip_recorded_lists=True, out=(lr_r, cnt_r, recs, rcnt))
    ws = torch.empty(lsa.attend_bucket_major_workspace_bytes(cache, cfg.H_q, cfg.d, 32768), dtype=torch.uint8,
                     device=DEV)
    tail = (cache, cfg.k, cfg.n_sinks, cfg.window)
    Ob = lsa.sparse_attend_bucket_major(Qc, G["K"], G["V"], qpc, lr_r, cnt_r, *tail, workspace=ws,
                                        bucket_records=(recs, rcnt))
    Ol = lsa.sparse_attend_bucket_major(Qc, G["K"], G["V"], qpc, lr, cnt, *tail, workspace=ws)
    del ws
    Og = lsa.sparse_attend(Qc, G["K"], G["V"], qpc, lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    assert torch.equal(cnt_r, cnt) and bool((rcnt >= 0).float().mean() > 0.99)
    assert torch.equal(Ob, Ol)
    d_gather = float((Ob.float() - Og.float()).abs().max())
    print(f"[1m] bench path (records, bucket-major) vs gather max abs diff {d_gather:.3e}", flush=True)
    assert d_gather <= tol_for("bf16")
    del Ob, Ol, Og, lr_r, recs
    # attention on synthetic lists for sampled late queries
    qs = torch.tensor(sorted(rng.integers(cfg.T - 4096, cfg.T, 64).tolist()), dtype=torch.int64)
    Qs = G["Q"][:, qs.to(DEV)].contiguous()
    qp = qs.unsqueeze(0).to(DEV)
    idx, ln = random_lr_lists(cfg, qs.unsqueeze(0), seed=3)
    Og = lsa.sparse_attend(Qs, G["K"], G["V"], qp, idx.to(DEV), ln.to(DEV), cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    err = 0.0
    for j, t in enumerate(qs.tolist()):
        for g in range(0, cfg.H_kv, 3):
            row = lr_row(idx[0, j, g].numpy(), int(ln[0, j, g]))
            S = np.union1d(np.union1d(np.arange(min(cfg.n_sinks, t + 1)),
                                      np.arange(O.query_geometry(t, cfg.T // 2048, cfg.n_sinks, cfg.window)[2], t + 1)),
                           row)
            Kr = G["K"][0, g, torch.from_numpy(S).to(DEV)].double().cpu().numpy()
            Vr = G["V"][0, g, torch.from_numpy(S).to(DEV)].double().cpu().numpy()
            qg = Qs[0, j, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
            ref = O.attend_set(qg, Kr, Vr, np.arange(len(S)), 1 / math.sqrt(cfg.d))
            err = max(err, float(np.max(np.abs(ref - Og[0, j, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()))))
    print(f"[1m] attend max abs err {err:.2e}", flush=True)
    assert err <= tol_for("bf16")


def test_decode_16x1m():
    cfg = get_config(3)
    print("[decode] generating", flush=True)
    inp = decode_inputs(cfg, seed=0, device=DEV)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], T=cfg.T, n_q_heads=cfg.H_q)
    lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    lr_c, cnt_c = lr.cpu().numpy(), cnt.cpu().numpy()
    rng = np.random.default_rng(5)
    W = G["W"].double().cpu().numpy()
    pairs = [(int(rng.integers(0, cfg.B)), int(rng.integers(0, cfg.H_kv)), int(rng.integers(0, cfg.T // 2048)))
             for _ in range(16)]
    ward = _sampled_ward(G["K"], W, cache, pairs)
    print("[decode] ward", ward, flush=True)
    assert ward["unexcused"] == 0 and ward["exact"] >= 14
    units = [(b, 0, g) for b in range(0, cfg.B, 3) for g in range(cfg.H_kv)]
    res = _sampled_fullsize(cfg, G, cache, lr_c, cnt_c, units,
                            q_of=lambda b, i, g: G["Q"][b, 0, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy(),
                            t_of=lambda b, i: cfg.T)
    print(f"[decode] select {res}", flush=True)
    assert res["unexcused"] == 0
    # attention (split-key path) on synthetic lists for every (sequence, KV head)
    idx, ln = random_lr_lists(cfg, torch.full((cfg.B, 1), cfg.T, dtype=torch.int64), seed=6)
    Og = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], idx.to(DEV), ln.to(DEV), cfg.T, cfg.k, cfg.n_sinks,
                           cfg.window)
    torch.cuda.synchronize()
    err = 0.0
    t = cfg.T
    l0 = O.query_geometry(t, cfg.T // 2048, cfg.n_sinks, cfg.window)[2]
    for b in range(cfg.B):
        for g in range(cfg.H_kv):
            row = lr_row(idx[b, 0, g].numpy(), int(ln[b, 0, g]))
            S = np.union1d(np.union1d(np.arange(cfg.n_sinks), np.arange(l0, t + 1)), row)
            Sd = torch.from_numpy(S).to(DEV)
            Kr = G["K"][b, g, Sd].double().cpu().numpy()
            Vr = G["V"][b, g, Sd].double().cpu().numpy()
            qg = G["Q"][b, 0, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
            ref = O.attend_set(qg, Kr, Vr, np.arange(len(S)), 1 / math.sqrt(cfg.d))
            err = max(err, float(np.max(np.abs(ref - Og[b, 0, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()))))
    print(f"[decode] attend max abs err {err:.2e}", flush=True)
    assert err <= tol_for("bf16")


def test_prefill_10m_tree_sampled():
    cfg = get_config(5)
    rng = np.random.default_rng(8)
    qs = torch.tensor(sorted(rng.integers(2048, cfg.T, 48).tolist()), dtype=torch.int64).unsqueeze(0)
    print("[10m] generating", flush=True)
    inp = layer_inputs(cfg, seed=0, device=DEV, q_positions=qs)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q, build_tree=True)
    lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, search="tree",
                         beam=cfg.beam)
    torch.cuda.synchronize()
    W = G["W"].double().cpu().numpy()
    pairs = [(0, int(rng.integers(0, cfg.H_kv)), int(rng.integers(0, cfg.T // 2048))) for _ in range(12)]
    ward = _sampled_ward(G["K"], W, cache, pairs)
    print("[10m] ward", ward, flush=True)
    assert ward["unexcused"] == 0 and ward["exact"] >= 11
    # tree nodes: normalised sums of their children, root unit norm
    c1, s1 = cache.tree_level(1)
    s0 = cache.sums()[0, 0]
    assert torch.allclose(s1[0, 0, :1000], s0[0:2000:2] + s0[1:2000:2], rtol=1e-5, atol=1e-5)
    lr_c, cnt_c = lr.cpu().numpy(), cnt.cpu().numpy()
    units = [(0, i, g) for i in range(0, qs.shape[1], 2) for g in (0, 5)]
    res = _sampled_fullsize(cfg, G, cache, lr_c, cnt_c, units, tree=True, beam=cfg.beam,
                            q_of=lambda b, i, g: G["Q"][b, i, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy(),
                            t_of=lambda b, i: int(qs[0, i]))
    print(f"[10m] tree select {res}", flush=True)
    assert res["unexcused"] == 0
    # bucket-major with the tree cache and the selection's records (lists skipped), as the bench times it:
    # equal to the same call on the lists, and to the gather call
    lr_r, cnt_r = torch.empty_like(lr), torch.empty_like(cnt)
    recs = torch.empty(*cnt.shape, 256, 4, dtype=torch.int32, device=DEV)
    rcnt = torch.empty_like(cnt)
    lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, search="tree", beam=cfg.beam,
               bucket_records=True, skip_recorded_lists=True, out=(lr_r, cnt_r, recs, rcnt))
    tail = (cache, cfg.k, cfg.n_sinks, cfg.window)
    Ob = lsa.sparse_attend_bucket_major(G["Q"], G["K"], G["V"], G["q_pos"], lr_r, cnt_r, *tail,
                                        bucket_records=(recs, rcnt))
    Ol = lsa.sparse_attend_bucket_major(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, *tail)
    Og = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    assert torch.equal(cnt_r, cnt) and torch.equal(Ob, Ol)
    d_gather = float((Ob.float() - Og.float()).abs().max())
    print(f"[10m] bucket-major (records) vs gather max abs diff {d_gather:.3e}", flush=True)
    assert d_gather <= tol_for("bf16")
