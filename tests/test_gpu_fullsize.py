"""Parity at the workloads' full sizes, in the launch configuration bench.py
times.

The oracle's inputs never come from the HIP path, except the bucket
membership, which is checked first: every block of the compared (sequence,
KV head) must be a valid partition (64 buckets of 1..16 entries covering the
block) and sampled blocks must match the oracle's own Ward on K (margin
protocol).  From K, W and that membership the oracle then recomputes every
leaf centroid (and at 10M every tree node) itself; the GPU's must lie within
one bf16 step of them (2^-16 for components below 2^-9).  Selections and outputs are the oracle's own, on its
own cache, against the GPU's.

* 131,072-token prefill (8 KV / 40 query heads): the oracle rebuilds the whole
  bucket cache from K (every Ward block) and recomputes sampled selections and
  outputs on its own.
* 1M prefill: the whole layer runs as the bench times it (65,536-query
  chunks: selection written as bucket records with the recorded rows' lists
  skipped, then bucket-major attention in passes of 32,768 queries, with zero
  rows gathered whole); 256 (query, KV head) units stratified over the blocks
  are compared: the records expanded on the host against the oracle's flat
  selection, the output against the oracle's attention.
* 16 x 1M decode: all 128 (sequence, KV head) units: caches, needle blocks'
  Ward, selection, output, and needle retrieval (the GPU finds the needle
  exactly where the oracle does).
* 10M tree prefill and the 8-query decode on its shared cache: the timed
  path on queries sampled over the blocks (each query's result is
  independent of the other queries of its pass), tree nodes recomputed by the
  oracle, selections by the oracle's tree search.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_indexing_latent_amd as lsa
from synth import decode_inputs, get_config, layer_inputs
from synth.topics import make_queries
from tests.parity import (MARGIN, centroid_excess, check_lr_wellformed, check_partitions, compare_ward,
                          expand_records, gpu_partitions, lr_row, tol_for, ward_first_divergence_margin)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CHUNK = 65536


def _oracle_head(K, W, cache, b, g, T, tree=False):
    """The oracle's cache of (b, g) on the GPU's membership (validated), and the GPU-vs-oracle centroid
    differences (leaves, then every tree level) over what rounding allows (centroid_excess).  Returns
    (cache dict, Kg float64 with every row of K, clusters, worst excess, centroids not bit-equal)."""
    clusters = gpu_partitions(cache, b, g)
    check_partitions(clusters)
    nb = T // 2048
    Kg = K[b, g].double().cpu().numpy()
    oc = O.build_head_cache(Kg, W, "bf16", T=nb * 2048, clusters=clusters, tree=tree)
    gc = cache.centroids()[b, g]
    d = centroid_excess(gc, oc["cent"])
    worst, diff = float(d.max()), int((gc.double().cpu().numpy() != oc["cent"]).any(axis=1).sum())
    if tree:
        info = cache.info()
        assert info.n_levels == len(oc["tree"])
        for lev in range(1, info.n_levels):
            c, _ = cache.tree_level(lev)
            dl = centroid_excess(c[b, g], oc["tree"][lev]["cent"])
            worst = max(worst, float(dl.max()))
            diff += int((c[b, g].double().cpu().numpy() != oc["tree"][lev]["cent"]).any(axis=1).sum())
    return oc, Kg, clusters, worst, diff


def _ward_sample(K, W, clusters, b, g, blocks, processes=16):
    """The oracle's own Ward on sampled blocks of (b, g) against the GPU partitions (margin protocol)."""
    E = []
    for blk in blocks:
        Kb = K[b, g, blk * 2048:(blk + 1) * 2048].double().cpu().numpy()
        E.append(O.pooled_entries(O.key_latents(Kb, W)))
    own = O.ward_blocks(E, processes=processes)
    st = dict(blocks=0, exact=0, excused=0, unexcused=0)
    for e, oc, blk in zip(E, own, blocks):
        st["blocks"] += 1
        gc = clusters[blk]
        if [list(c) for c in oc] == gc:
            st["exact"] += 1
        elif ward_first_divergence_margin(e, gc) < MARGIN:
            st["excused"] += 1
        else:
            st["unexcused"] += 1
    return st


def _judge(run, got):
    """run(with_margin) -> (list, info) is the oracle's selection; its margin (a scan of every visible
    leaf, slow at 10M) is taken only when the lists differ."""
    ref, _ = run(False)
    if np.array_equal(ref, got):
        return "exact", ref
    ref, info = run(True)
    return ("excused" if info["margin"] < MARGIN else "unexcused"), ref


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


def _prefill_path(Q, q_pos, K, V, W, cache, cfg, n_pass, O_out, want, search="flat", beam=0):
    """The bench's timed prefill path over all of Q (chunks of whole passes): select with bucket records
    and the recorded rows' lists skipped, then bucket-major attention with a workspace for n_pass
    queries.  Returns the fallback counts and, for the wanted (query index, g), the records and counts."""
    n_q = Q.shape[1]
    chunk = n_pass * max(1, CHUNK // n_pass)
    ws = torch.empty(lsa.attend_bucket_major_workspace_bytes(cache, cfg.H_q, cfg.d, min(n_pass, n_q)),
                     dtype=torch.uint8, device=DEV)
    fc = torch.zeros(2, dtype=torch.int32, device=DEV)
    got = {}
    for i0 in range(0, n_q, chunk):
        i1 = min(n_q, i0 + chunk)
        lr, cnt, (recs, rcnt) = lsa.select(Q[:, i0:i1], cache, q_pos[:, i0:i1], W, cfg.k, cfg.n_sinks, cfg.window,
                                           search=search, beam=beam, strategy="fused" if search == "flat" else "auto",
                                           bucket_records=True, skip_recorded_lists=True)
        lsa.sparse_attend_bucket_major(Q[:, i0:i1], K, V, q_pos[:, i0:i1], lr, cnt, cache, cfg.k, cfg.n_sinks,
                                       cfg.window, O=O_out[:, i0:i1], workspace=ws, bucket_records=(recs, rcnt),
                                       fallback_counts=fc)
        mine = [(i, g) for (i, g) in want if i0 <= i < i1]
        if mine:
            ii = torch.tensor([i - i0 for i, _ in mine], device=DEV)
            gg = torch.tensor([g for _, g in mine], device=DEV)
            r_c, n_c, c_c = recs[0, ii, gg].cpu().numpy(), rcnt[0, ii, gg].cpu().numpy(), cnt[0, ii, gg].cpu().numpy()
            l_c = lr[0, ii, gg].cpu().numpy()
            for j, key in enumerate(mine):
                got[key] = (r_c[j], int(n_c[j]), int(c_c[j]), l_c[j])
        del lr, cnt, recs, rcnt
    torch.cuda.synchronize()
    return fc.tolist(), got


def _check_units(cfg, units, ocs, got, Qh, O_h, t_of, search, beam, tag):
    """units: (query index, g).  The GPU's records, expanded on the host with the (validated) membership,
    against the oracle's selection on its own cache; the output rows against the oracle's attention."""
    W = ocs["W"]
    scale = 1 / math.sqrt(cfg.d)
    res = dict(exact=0, excused=0, unexcused=0)
    err = 0.0
    listed = 0
    for (i, g) in units:
        oc, Kg, Vg = ocs[g]
        t = t_of(i)
        qg = Qh(i, g)
        qh = O.query_latent(qg, W, "bf16")
        recs, n, cnt, lrow = got[(i, g)]
        if n >= 0:
            row = expand_records(recs, n, oc["members"])
        else:   # a row the selection did not record (trivial, or the exact fallback) has its list written
            row = lr_row(lrow, cnt)
            listed += 1
        assert len(row) == cnt
        check_lr_wellformed(row, cfg.k, t, oc["n_blocks"], cfg.n_sinks, cfg.window, cnt, flat=search == "flat")
        if search == "flat":
            run = lambda wm: O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, with_margin=wm)
        else:
            run = lambda wm: O.select_tree(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window, beam, with_margin=wm)
        res[_judge(run, row)[0]] += 1
        out = O.attend(qg, Kg, Vg, t, row, cfg.n_sinks, cfg.window, oc["n_blocks"], scale)
        err = max(err, float(np.max(np.abs(out - O_h(i, g)))))
        if sum(res.values()) % 64 == 0:
            print(f"[{tag}] {sum(res.values())}/{len(units)} units: {res}", flush=True)
    print(f"[{tag}] select {res} ({listed} rows without records) attend max abs err {err:.2e}", flush=True)
    assert res["unexcused"] == 0 and res["exact"] >= 0.9 * len(units)
    assert err <= tol_for("bf16")


def test_prefill_1m_oracle_on_the_timed_path():
    cfg = get_config(4)
    print("[1m] generating", flush=True)
    inp = layer_inputs(cfg, seed=0, device=DEV)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    del inp
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q)
    rng = np.random.default_rng(4)
    heads = sorted(rng.choice(cfg.H_kv, 2, replace=False).tolist())
    # 128 units per head, stratified over the blocks
    edges = np.linspace(2048, cfg.T, 129)
    units = [(int(rng.integers(edges[j], edges[j + 1])), g) for g in heads for j in range(128)]
    Og = torch.empty_like(G["Q"])
    print("[1m] timed path over the whole layer", flush=True)
    fc, got = _prefill_path(G["Q"], G["q_pos"], G["K"], G["V"], G["W"], cache, cfg, 32768, Og, units)
    print(f"[1m] rows gathered whole: {fc}", flush=True)
    assert fc == [0, 0]
    W = G["W"].double().cpu().numpy()
    ocs = {"W": W}
    for g in heads:
        oc, Kg, clusters, worst, diff = _oracle_head(G["K"], W, cache, 0, g, cfg.T)
        print(f"[1m] g={g}: {len(oc['cent'])} centroids, {diff} not bit-equal, worst excess {worst:.3f}", flush=True)
        assert worst <= 1
        blocks = sorted(rng.choice(cfg.T // 2048, 12, replace=False).tolist())
        st = _ward_sample(G["K"], W, clusters, 0, g, blocks)
        print(f"[1m] g={g} ward {st}", flush=True)
        assert st["unexcused"] == 0 and st["exact"] >= 11
        ocs[g] = (oc, Kg, G["V"][0, g].double().cpu().numpy())
    Qh = lambda i, g: G["Q"][0, i, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
    O_h = lambda i, g: Og[0, i, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
    _check_units(cfg, units, ocs, got, Qh, O_h, lambda i: i, "flat", 0, "1m")


def test_decode_16x1m_every_unit():
    cfg = get_config(3)
    print("[decode] generating", flush=True)
    inp = decode_inputs(cfg, seed=0, device=DEV)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], T=cfg.T, n_q_heads=cfg.H_q)
    # the bench's decode step (the new token's K/V sit in row T)
    lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window)
    Og = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    lr_c, cnt_c, O_c = lr.cpu().numpy(), cnt.cpu().numpy(), Og.double().cpu().numpy()
    W = G["W"].double().cpu().numpy()
    t = cfg.T
    scale = 1 / math.sqrt(cfg.d)
    res = dict(exact=0, excused=0, unexcused=0)
    worst, diff, err = 0.0, 0, 0.0
    needle = dict(gpu=0, oracle=0, agree=0)
    misses = []
    E_needle, C_needle = [], []
    for b in range(cfg.B):
        p = inp["needle_pos"][b]
        for g in range(cfg.H_kv):
            oc, Kt, clusters, w, dd = _oracle_head(G["K"], W, cache, b, g, cfg.T)
            worst, diff = max(worst, w), diff + dd
            blk = p // 2048
            E_needle.append(oc["entries"][blk * 512:(blk + 1) * 512])
            C_needle.append(clusters[blk])
            qg = G["Q"][b, 0, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
            qh = O.query_latent(qg, W, "bf16")
            row = lr_row(lr_c[b, 0, g], int(cnt_c[b, 0, g]))
            check_lr_wellformed(row, cfg.k, t, oc["n_blocks"], cfg.n_sinks, cfg.window, int(cnt_c[b, 0, g]))
            verdict, ref = _judge(lambda wm: O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window,
                                                           with_margin=wm), row)
            res[verdict] += 1
            ref, info = O.select_flat(qh, oc, t, cfg.k, cfg.n_sinks, cfg.window)   # scores, for the needle
            Vg = G["V"][b, g].double().cpu().numpy()
            out = O.attend(qg, Kt, Vg, t, row, cfg.n_sinks, cfg.window, oc["n_blocks"], scale)
            err = max(err, float(np.max(np.abs(out - O_c[b, 0, g * cfg.G:(g + 1) * cfg.G]))))
            want = set(range(p, p + 4))
            f_gpu, f_ora = want <= set(row.tolist()), want <= set(ref.tolist())
            needle["gpu"] += f_gpu
            needle["oracle"] += f_ora
            needle["agree"] += f_gpu == f_ora
            if not f_ora:
                # why the method misses it: the needle's bucket, its size and where it ranks
                e = (p // 4) % 512
                leaf = blk * 64 + next(r for r, c in enumerate(clusters[blk]) if e in c)
                s = info["scores"]
                rank = int(np.sum((s > s[leaf]) | ((s == s[leaf]) & (np.arange(len(s)) < leaf))))
                bnd = info["boundary"]
                misses.append((b, g, len(oc["members"][leaf]), rank, float(s[leaf]), float(s[bnd])))
            del oc, Vg, Kt
        print(f"[decode] sequence {b}: {res}", flush=True)
    print(f"[decode] centroids: {diff} of {128 * 32768} not bit-equal, worst excess {worst:.3f}", flush=True)
    print(f"[decode] select {res} attend max abs err {err:.2e}", flush=True)
    print(f"[decode] needle found: GPU {needle['gpu']}/128, oracle {needle['oracle']}/128, "
          f"agree {needle['agree']}/128", flush=True)
    if misses:
        sizes = np.array([m[2] for m in misses])
        ranks = np.array([m[3] for m in misses])
        gap = np.array([m[5] - m[4] for m in misses])
        print(f"[decode] needle misses: bucket entries {np.bincount(sizes).tolist()} (count per size), "
              f"rank median {int(np.median(ranks))} (min {int(ranks.min())}), score below the boundary: "
              f"median {np.median(gap):.3f} (min {gap.min():.3f})", flush=True)
    # the needle blocks: the oracle's own Ward against the GPU partitions
    own = O.ward_blocks(E_needle, processes=16)
    wst = dict(exact=0, excused=0, unexcused=0)
    for e, oc_, gc in zip(E_needle, own, C_needle):
        if [list(c) for c in oc_] == gc:
            wst["exact"] += 1
        else:
            wst["excused" if ward_first_divergence_margin(e, gc) < MARGIN else "unexcused"] += 1
    print(f"[decode] needle blocks ward {wst}", flush=True)
    assert worst <= 1
    assert wst["unexcused"] == 0
    assert res["unexcused"] == 0 and res["exact"] >= 120
    assert err <= tol_for("bf16")
    assert needle["agree"] == 128


def test_prefill_10m_tree_and_decode():
    cfg = get_config(5)
    rng = np.random.default_rng(8)
    edges = np.linspace(2048, cfg.T, 129)
    qs = torch.tensor([int(rng.integers(edges[j], edges[j + 1])) for j in range(128)], dtype=torch.int64)
    print("[10m] generating", flush=True)
    inp = layer_inputs(cfg, seed=0, device=DEV, T_cap=cfg.T + 1, q_positions=qs.unsqueeze(0))
    # the decode token at row T, as the bench's decode step on this cache places it
    gen = torch.Generator(device=DEV)
    gen.manual_seed(12345)
    kn = torch.randn(cfg.B, cfg.H_kv, cfg.d, generator=gen, device=DEV)
    inp["K"][:, :, cfg.T] = (kn / kn.norm(dim=-1, keepdim=True)).to(inp["K"].dtype)
    inp["V"][:, :, cfg.T] = torch.randn(cfg.B, cfg.H_kv, cfg.d, generator=gen, device=DEV).to(inp["V"].dtype)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], T=cfg.T, n_q_heads=cfg.H_q, build_tree=True)
    heads = [0, 5]
    units = [(i, g) for g in heads for i in range(qs.numel())]
    Og = torch.empty_like(G["Q"])
    fc, got = _prefill_path(G["Q"], G["q_pos"], G["K"], G["V"], G["W"], cache, cfg, 40960, Og, units,
                            search="tree", beam=cfg.beam)
    print(f"[10m] rows gathered whole: {fc}", flush=True)
    assert fc == [0, 0]
    # decode: 8 queries at position T on the shared cache, tree search, split-key gather attention
    qp = torch.full((1, cfg.decode_batch), cfg.T, dtype=torch.int64)
    Qd = make_queries(cfg, 7, inp["mu"], inp["topic"], qp, DEV).contiguous()
    qp = qp.to(DEV)
    lrd, cntd = lsa.select(Qd, cache, qp, G["W"], cfg.k, cfg.n_sinks, cfg.window, search="tree", beam=cfg.beam)
    Od = lsa.sparse_attend(Qd, G["K"], G["V"], qp, lrd, cntd, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    W = G["W"].double().cpu().numpy()
    ocs = {"W": W}
    for g in heads:
        oc, Kg, clusters, worst, diff = _oracle_head(G["K"], W, cache, 0, g, cfg.T, tree=True)
        n_nodes = sum(len(lv["cent"]) for lv in oc["tree"])
        print(f"[10m] g={g}: {n_nodes} leaf and node centroids, {diff} not bit-equal, worst excess {worst:.3f}",
              flush=True)
        assert worst <= 1
        blocks = sorted(rng.choice(cfg.T // 2048, 12, replace=False).tolist())
        st = _ward_sample(G["K"], W, clusters, 0, g, blocks)
        print(f"[10m] g={g} ward {st}", flush=True)
        assert st["unexcused"] == 0 and st["exact"] >= 11
        ocs[g] = (oc, Kg, G["V"][0, g].double().cpu().numpy())
    Qh = lambda i, g: G["Q"][0, i, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
    O_h = lambda i, g: Og[0, i, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
    _check_units(cfg, units, ocs, got, Qh, O_h, lambda i: int(qs[i]), "tree", cfg.beam, "10m")
    # the decode leg
    lr_c, cnt_c, Od_c = lrd.cpu().numpy(), cntd.cpu().numpy(), Od.double().cpu().numpy()
    res = dict(exact=0, excused=0, unexcused=0)
    err = 0.0
    scale = 1 / math.sqrt(cfg.d)
    for g in heads:
        oc, Kt, Vt = ocs[g]
        for i in range(cfg.decode_batch):
            qg = Qd[0, i, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
            qh = O.query_latent(qg, W, "bf16")
            row = lr_row(lr_c[0, i, g], int(cnt_c[0, i, g]))
            check_lr_wellformed(row, cfg.k, cfg.T, oc["n_blocks"], cfg.n_sinks, cfg.window, int(cnt_c[0, i, g]),
                                flat=False)
            res[_judge(lambda wm: O.select_tree(qh, oc, cfg.T, cfg.k, cfg.n_sinks, cfg.window, cfg.beam,
                                                with_margin=wm), row)[0]] += 1
            out = O.attend(qg, Kt, Vt, cfg.T, row, cfg.n_sinks, cfg.window, oc["n_blocks"], scale)
            err = max(err, float(np.max(np.abs(out - Od_c[0, i, g * cfg.G:(g + 1) * cfg.G]))))
    print(f"[10m decode] select {res} attend max abs err {err:.2e}", flush=True)
    assert res["unexcused"] == 0 and res["exact"] >= 14
    assert err <= tol_for("bf16")
