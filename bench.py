#!/usr/bin/env python3
"""Benchmark of the LSA layer hot path on one MI355X.

Default workload: one bf16 prefill layer at T = 1,048,576 (8 KV / 40 query
heads, head_dim 128, 4096-topic mixture, k = 2048, 4 sinks, window 1024,
flat search).  One step = build_buckets over all keys + select and
sparse_attend for every query (in chunks of whole bucket-major passes), with
K, V, Q and W already resident in HBM.  The same run then measures the
decode step at 1M context (16 sequences, one query each, as HIP-graph
replays), and the 10M-token tree layer (16,384 topics, beam 64; a fixed
--steps-10m timed steps after --warmup-10m) with its 8-query decode step on
the shared cache, each under its own key of the one JSON line.

Prints one JSON line (metric, value = the 1M layer's tokens/s, roofline of
the dominant call measured with HIP events on the launch stream, and the CPU
oracle baseline timed on a bounded sample).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_attention_indexing_latent_amd as lsa  # noqa: E402
from synth import decode_inputs, get_config, layer_inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0
CHUNK = 65536


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP events on the current (launch) stream."""

    def __init__(self):
        self.pairs = []

    def span(self):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        self.pairs.append((s, e))
        return e

    def total_ms(self):
        return sum(s.elapsed_time(e) for s, e in self.pairs)

    def count(self):
        return len(self.pairs)


def prefill_step(cfg, G, ws, timers=None, tree=False, O=None):
    """One pass of the whole hot path over one layer."""
    tm = timers
    if tm:
        e = tm["build"].span()
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q, build_tree=tree, cache=ws.get("cache"))
    ws["cache"] = cache.buf
    if tm:
        e.record()
    n_q = G["Q"].shape[1]
    chunk = ws.get("chunk", CHUNK)
    for i0 in range(0, n_q, chunk):
        i1 = min(n_q, i0 + chunk)
        Qc = G["Q"][:, i0:i1]
        qp = G["q_pos"][:, i0:i1]
        if tm:
            e = tm["select"].span()
        recs = "recs" in ws
        # rows with records need no token list, except in the step that counts the algorithmic bytes
        skip = recs and ws.get("skip_lists", False) and "cnt_sum" not in ws
        res = lsa.select(Qc, cache, qp, G["W"], cfg.k, cfg.n_sinks, cfg.window,
                         search="tree" if tree else "flat", beam=cfg.beam, workspace=ws.get("sel"),
                         out=(ws["lr"][:, : i1 - i0], ws["cnt"][:, : i1 - i0])
                         + ((ws["recs"][:, : i1 - i0], ws["rcnt"][:, : i1 - i0]) if recs else ()),
                         bucket_records=recs, skip_recorded_lists=skip)
        lr, cnt = res[0], res[1]
        if tm:
            e.record()
            e = tm["attend"].span()
        if "bm" in ws:
            lsa.sparse_attend_bucket_major(Qc, G["K"], G["V"], qp, lr, cnt, cache, cfg.k, cfg.n_sinks, cfg.window,
                                           O=O[:, i0:i1], workspace=ws["bm"], bucket_records=res[2] if recs else None,
                                           fallback_counts=ws.get("fallback"))
        else:
            lsa.sparse_attend(Qc, G["K"], G["V"], qp, lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window,
                              O=O[:, i0:i1])
        if tm:
            e.record()
        if "cnt_sum" in ws:
            ws["cnt_sum"] += int(cnt.clamp_min(0).sum().item())
            if "bm" in ws:
                ws["bm_bytes"] += bucket_major_bytes(cfg, lr, cnt, cache, ws["bm_pass"], records="recs" in ws)
    return cache


def selected_bytes(cfg, n_q_total, lr_total, q_pos_all, tile=64):
    """Algorithmic HBM bytes of the gather attention over all queries.

    Every long-range key and value row of every (query, KV head), once; the
    sink and local-window rows once per tile of 64 consecutive queries of a
    KV head (consecutive windows overlap, so a tile needs the union of its
    windows); Q read and O written once.  Rows are head_dim bf16 values."""
    t = q_pos_all.double()
    nvis = torch.clamp(torch.div(t, 2048, rounding_mode="floor"), max=cfg.T // 2048)
    l0 = torch.clamp(torch.minimum(t - cfg.window + 1, 2048 * nvis), min=0)
    first = torch.arange(0, len(t), tile)
    last = torch.clamp(first + tile - 1, max=len(t) - 1)
    local_rows = float((t[last] - l0[first] + 1 + torch.clamp(l0[first], max=cfg.n_sinks)).sum())
    row = cfg.d * 2
    keys = local_rows * cfg.H_kv + lr_total
    return keys * 2 * row + 2 * n_q_total * cfg.H_q * row


def bucket_major_bytes(cfg, lr, cnt, cache, n_pass, sub=2048, records=False):
    """Algorithmic HBM bytes of one bucket-major attention call over a chunk
    of queries, without the window part (added by selected_bytes' local term):
    per pass, the K and V rows of every distinct bucket any of its queries
    listed, once; per (query, KV head, bucket) pair, the G query rows and
    the partial row (G x (2 d + 16) bytes: fp16 values, max, denominator,
    scale) written once and read once; the long-range lists read once, or
    with the selection's bucket records one 16-byte record per pair
    instead."""
    info = cache.info()
    nb = info.n_blocks
    eleaf = cache.entry_leaf()[0].long()                     # [H_kv, nb, 512]
    size = (cache.meta()[0].long() & 0xFF)                   # [H_kv, n_leaves]
    H, k, d, G = cfg.H_kv, cfg.k, cfg.d, cfg.G
    nq = lr.shape[1]
    pairs, kv_rows = 0, 0
    gidx = torch.arange(H, device=lr.device).view(1, H, 1)
    for p0 in range(0, nq, n_pass):
        seen = []
        for s0 in range(p0, min(nq, p0 + n_pass), sub):
            s1 = min(nq, p0 + n_pass, s0 + sub)
            L = lr[0, s0:s1].long()                           # [n, H, k]
            valid = torch.arange(k, device=L.device).view(1, 1, k) < cnt[0, s0:s1].unsqueeze(-1)
            tok = torch.where(valid, L, torch.zeros_like(L))
            blk = torch.clamp(tok // 2048, max=max(nb - 1, 0))
            rank = eleaf[gidx, blk, (tok // 4) % 512]
            key = torch.where(valid, gidx * (nb * 64) + blk * 64 + rank, torch.full_like(L, -1))
            srt = key.sort(dim=-1).values
            new = (srt[..., 1:] != srt[..., :-1]) & (srt[..., 1:] >= 0)
            pairs += int(new.sum()) + int((srt[..., 0] >= 0).sum())
            seen.append(torch.unique(srt[srt >= 0]))
        if seen:
            u = torch.unique(torch.cat(seen))
            kv_rows += int((size.view(-1)[u] * 4).sum())
    row = d * 2
    lists = pairs * 16 if records else int(cnt.clamp_min(0).sum()) * 4
    return kv_rows * 2 * row + pairs * G * row + 2 * pairs * G * (2 * d + 16) + lists


_CPU_CTX = {}


def _cpu_units(items):
    """select + attend of the oracle for a list of (position, query rows) (one process, one BLAS thread)."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    c = _CPU_CTX
    cfg, cache, Kg, Vg, W = c["cfg"], c["cache"], c["Kg"], c["Vg"], c["W"]
    scale = 1 / math.sqrt(cfg.d)
    with threadpool_limits(1):
        for t, qg in items:
            qh = O.query_latent(qg, W, cfg.dtype)
            if cfg.search == "tree":
                lr, _ = O.select_tree(qh, cache, int(t), cfg.k, cfg.n_sinks, cfg.window, cfg.beam)
            else:
                lr, _ = O.select_flat(qh, cache, int(t), cfg.k, cfg.n_sinks, cfg.window)
            O.attend(qg, Kg, Vg, int(t), lr, cfg.n_sinks, cfg.window, cache["n_blocks"], scale)
    return len(items)


def cpu_baseline(cfg, inp_cpu, n_units=1500):
    """Oracle timed on this host: Ward on every block of KV head 0 of a CPU-generated layer, and
    select + attend for n_units (query, KV head) units against the oracle's own cache of those
    blocks, both spread over one process per core; the full-layer time is projected from the
    measured per-unit costs."""
    import oracle as O

    cores = len(os.sched_getaffinity(0))
    procs = max(1, min(cores, 16))
    nb = inp_cpu["K"].shape[2] // 2048
    Kg = inp_cpu["K"][0, 0, : nb * 2048].double().numpy()
    W = inp_cpu["W"].double().numpy()
    e = O.pooled_entries(O.key_latents(Kg, W))
    blocks = [e[b * 512:(b + 1) * 512] for b in range(nb)]
    t0 = time.perf_counter()
    clusters = O.ward_blocks(blocks, processes=procs)
    t_ward = time.perf_counter() - t0
    tree = cfg.search == "tree"
    cache = O.build_head_cache(Kg, W, cfg.dtype, T=nb * 2048, clusters=clusters, tree=tree)
    _CPU_CTX.update(cfg=cfg, cache=cache, Kg=Kg, Vg=inp_cpu["V"][0, 0, : nb * 2048].double().numpy(), W=W)
    rng = np.random.default_rng(0)
    ts = rng.integers((nb - 1) * 2048, nb * 2048, n_units)
    items = [(int(t), inp_cpu["Q"][0, int(t), : cfg.G].double().numpy()) for t in ts]   # plain arrays before forking
    parts = [items[i::procs] for i in range(procs)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(procs) as pool:
        pool.map(_cpu_units, parts)
    t_units = time.perf_counter() - t0
    # full-layer projection: Ward per block, and select + attend per (query, KV head) unit; flat
    # selection cost grows with the visible buckets, tree selection with the depth
    leaves_sample = (nb - 1) * 64
    mean_leaves = 64 * (cfg.T // 2048 - 1) / 2
    if tree:
        leaves_sample, mean_leaves = math.log2(max(2, leaves_sample)), math.log2(max(2, mean_leaves))
    wall_per_block = t_ward / nb                 # with procs processes
    wall_per_unit = t_units / n_units
    full_s = (cfg.T // 2048) * cfg.H_kv * wall_per_block + \
        cfg.T * cfg.H_kv * wall_per_unit * max(1.0, mean_leaves / leaves_sample)
    return dict(value=cfg.T / full_s, unit="tokens/s", cores=cores, processes=procs, kind="oracle",
                sample=(f"the same topic-mixture recipe generated on the CPU at T={nb * 2048}: oracle Ward on its {nb} "
                        f"blocks of KV head 0 ({t_ward:.1f}s wall) and select+attend for {n_units} (query, KV head) "
                        f"units at {(nb - 1) * 64} visible buckets ({t_units:.1f}s wall), each spread over {procs} "
                        f"processes ({(t_ward + t_units) * procs:.0f} core-seconds); full 1-layer time projected as "
                        f"blocks*H_kv*t_block + T*H_kv*t_unit*(mean visible buckets / sampled)"))


def traffic_for(kernel_src, key: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE, if
    they were taken on the current kernel source (one file, or a list whose
    contents are hashed in order)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(key)
    except Exception:
        return None
    if not rec:
        return None
    srcs = [kernel_src] if isinstance(kernel_src, str) else list(kernel_src)
    hs = hashlib.sha256()
    for f in srcs:
        hs.update(open(f, "rb").read())
    h = hs.hexdigest()
    return rec.get("bytes_per_launch") if rec.get("source_sha256") == h else None


def run_prefill(args, cid, steps, warmup):
    cfg = get_config(cid)
    dev = torch.device("cuda:0")
    log(f"generating {cfg.name} on the GPU")
    # one spare K/V row at position T serves the decode step on the same cache
    inp = layer_inputs(cfg, seed=0, device=dev, T_cap=cfg.T + 1)
    g = torch.Generator(device=dev)
    g.manual_seed(12345)
    kn = torch.randn(cfg.B, cfg.H_kv, cfg.d, generator=g, device=dev)
    inp["K"][:, :, cfg.T] = (kn / kn.norm(dim=-1, keepdim=True)).to(inp["K"].dtype)
    inp["V"][:, :, cfg.T] = torch.randn(cfg.B, cfg.H_kv, cfg.d, generator=g, device=dev).to(inp["V"].dtype)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    torch.cuda.synchronize()
    n_q = G["Q"].shape[1]
    ws = {"lr": torch.empty(1, CHUNK, cfg.H_kv, cfg.k, dtype=torch.int32, device=dev),
          "cnt": torch.empty(1, CHUNK, cfg.H_kv, dtype=torch.int32, device=dev)}
    tree = cfg.search == "tree"
    O = torch.empty_like(G["Q"])
    # workspace sized for the largest chunk
    cache0 = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q, build_tree=tree)
    nbytes = lsa.select_workspace_bytes(cache0, lsa.select_cfg(cfg.k, cfg.n_sinks, cfg.window,
                                                               "tree" if tree else "flat", cfg.beam),
                                        min(CHUNK, n_q), cfg.H_q)
    ws["sel"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws["cache"] = cache0.buf
    attend = args.attend if cfg.dtype == "bf16" else "gather"   # the bucket-major call is bf16 only
    ws["fallback"] = torch.zeros(2, dtype=torch.int32, device=dev)
    if attend != "gather" and args.bucket_records != "off":
        ws["skip_lists"] = args.bucket_records == "only"
        # the selection's bucket records for the bucket-major attention (one chunk's worth)
        ws["recs"] = torch.empty(1, CHUNK, cfg.H_kv, lsa._lib.BUCKET_RECS, 4, dtype=torch.int32, device=dev)
        ws["rcnt"] = torch.empty(1, CHUNK, cfg.H_kv, dtype=torch.int32, device=dev)
    if attend != "gather":
        # passes of up to --bm-pass queries, fewer (in steps of 4096) if free memory is short (workspace <= --bm-mem of it)
        torch.cuda.empty_cache()
        free = torch.cuda.mem_get_info(dev)[0]
        # default start: 32768 queries when such a pass gives each listed bucket >= 8 pairs on average (its
        # K/V reads already shared: measured equal or better than larger passes at 1M), else 65536 (at 10M a
        # bucket gets ~6 pairs per 32768 queries; 40960-query passes, the most that fit, were 7% faster)
        n_pass = args.bm_pass or (32768 if 32768 * cfg.k >= 8 * cfg.T else 65536)
        while n_pass > 4096 and lsa.attend_bucket_major_workspace_bytes(cache0, cfg.H_q, cfg.d, n_pass) > args.bm_mem * free:
            n_pass -= 4096
        # auto: bucket-major when a bucket is expected in >= 2 pairs per pass (n_pass * k / T); measured:
        # ahead of the gather at 1M (64 per pass) and at 10M (3.2 per pass: 8.7 s vs 14.0 s per layer)
        if attend == "auto":
            attend = "bucket" if n_pass * cfg.k >= 2 * cfg.T else "gather"
        if attend == "bucket":
            ws["bm"] = torch.empty(lsa.attend_bucket_major_workspace_bytes(cache0, cfg.H_q, cfg.d, n_pass),
                                   dtype=torch.uint8, device=dev)
            ws["bm_pass"] = n_pass
            # query chunks of whole passes (each select call feeds one attention call)
            ws["chunk"] = n_pass * max(1, CHUNK // n_pass)
            log(f"bucket-major attention, passes of {n_pass} queries, chunks of {ws['chunk']}, "
                f"workspace {ws['bm'].numel() / 2**30:.1f} GiB")
    if attend == "gather":
        log("gather attention")
        ws.pop("recs", None)
        ws.pop("rcnt", None)
        ws.pop("skip_lists", None)
    ws["cnt_sum"] = 0
    ws["bm_bytes"] = 0
    log(f"warmup ({warmup} steps)")
    for _ in range(warmup):
        ws["cnt_sum"] = 0
        ws["bm_bytes"] = 0
        prefill_step(cfg, G, ws, tree=tree, O=O)
    lr_total = ws.pop("cnt_sum") if warmup > 0 else None
    torch.cuda.synchronize()
    timers = {k: Timer() for k in ("build", "select", "attend")}
    log(f"timing {steps} steps")
    t0 = time.perf_counter()
    torch.cuda.synchronize()
    for _ in range(steps):
        prefill_step(cfg, G, ws, timers, tree=tree, O=O)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if lr_total is None:
        ws["cnt_sum"] = 0
        ws["bm_bytes"] = 0
        prefill_step(cfg, G, ws, tree=tree, O=O)
        lr_total = ws.pop("cnt_sum")
    fallbacks = ws["fallback"].tolist()
    n_runs = steps + (warmup if warmup > 0 else 1)   # warm-up steps, or the one step that counts the bytes
    ms_step = wall * 1000 / steps
    att_ms = timers["attend"].total_ms() / steps
    n_att = timers["attend"].count() // steps
    csrc = os.path.join(ROOT, "sparse_attention_indexing_latent_amd", "csrc")
    if attend == "bucket":
        # the window part as in the gather accounting, with no long-range rows
        alg_bytes = selected_bytes(cfg, n_q, 0, G["q_pos"][0].cpu()) + ws["bm_bytes"]
        kernel = f"bucket-major attention call (pairs, scan, scatter, bm_leaf_kernel<{cfg.d}>, bm_local_kernel<{cfg.d}>)"
        traffic = traffic_for([os.path.join(csrc, "lsa_bucket.hip"), os.path.join(csrc, "lsa_attend.hip")],
                              f"attend_bucket_{cfg.name}")
    else:
        alg_bytes = selected_bytes(cfg, n_q, lr_total, G["q_pos"][0].cpu())
        kernel = f"attend_bf16_kernel<{cfg.d}>" if cfg.dtype == "bf16" else "attend_f32_kernel"
        traffic = traffic_for(os.path.join(csrc, "lsa_attend.hip"), f"attend_{cfg.name}")
    achieved = alg_bytes / (att_ms / 1e3) / 1e9
    per_launch = alg_bytes / n_att
    res = dict(
        metric="1-layer LSA prefill tokens/s at 1M & 10M ctx; decode queries/s at 1M (1 GPU)",
        value=cfg.T / (ms_step / 1e3), unit="tokens/s", n_gpus=1, steps=steps, warmup=warmup,
        ms_per_step=ms_step, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16" if cfg.dtype == "bf16" else "f32",
        data="synthetic (seeded topic-mixture keys, random-init projection)",
        config={"workload": cfg.name, "T": cfg.T, "H_kv": cfg.H_kv, "H_q": cfg.H_q, "head_dim": cfg.d,
                "k": cfg.k, "n_sinks": cfg.n_sinks, "window": cfg.window, "search": cfg.search,
                "beam": cfg.beam, "query_chunk": ws.get("chunk", CHUNK), "attention": attend,
                "bucket_pass": ws.get("bm_pass"),
                "bucket_records": ("only" if ws.get("skip_lists") else "on") if "recs" in ws else "off"},
        breakdown_ms={"build_buckets": timers["build"].total_ms() / steps,
                      "select": timers["select"].total_ms() / steps, "sparse_attend": att_ms},
        roofline={"kernel": kernel, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                  "traffic": traffic, "alg_bytes_per_launch": per_launch,
                  "avg_launch_ms": att_ms / n_att, "launches_per_step": n_att},
    )
    if attend == "bucket":
        # (query, KV head) rows the bucket-major call gathered whole, over every step run (warm-up included),
        # and of those the rows whose pairs did not fit in a pass's pool
        res["bucket_major_fallbacks"] = {"rows": fallbacks[0], "pool_full": fallbacks[1], "steps_run": n_runs}
    if cfg.decode_batch:
        res["decode_shared"] = decode_on_cache(cfg, G, inp, ws["cache"], tree)
    return res, cfg, inp


def kv_rows(K, T):
    """Flat row index of position T for every (sequence, KV head) of K [B, H_kv, t_cap, d]."""
    B, H, t_cap, _ = K.shape
    return torch.arange(B * H, device=K.device) * t_cap + T


def pair_kv(G):
    """Move K and V into one allocation [2, B, H_kv, t_cap, d] (K = [0], V = [1]) so that a decode
    step appends both rows with one index_copy_; returns that tensor."""
    KV = torch.empty((2,) + tuple(G["K"].shape), dtype=G["K"].dtype, device=G["K"].device)
    KV[0].copy_(G["K"])
    KV[1].copy_(G["V"])
    G["K"], G["V"] = KV[0], KV[1]
    return KV


def append_kv_pair(KV, rows2, newKV):
    """Both rows of the new token into the paired K/V tensor with one index_copy_ (rows2: the K rows,
    then the same rows of V)."""
    KV.view(-1, KV.shape[-1]).index_copy_(0, rows2, newKV)


def append_kv(G, rows, newK, newV):
    """Write one new token's key/value rows: one index_copy_ per tensor (a
    slice assignment into a >2^31-element tensor splits into one copy per
    sequence)."""
    d = G["K"].shape[-1]
    G["K"].view(-1, d).index_copy_(0, rows, newK.reshape(-1, d))
    G["V"].view(-1, d).index_copy_(0, rows, newV.reshape(-1, d))


def decode_on_cache(cfg, G, inp, cache_buf, tree):
    """decode_batch queries at position T on the layer's own cache (the new
    token's K/V sits in row T)."""
    from synth.topics import make_queries
    dev = G["K"].device
    nq = cfg.decode_batch
    qp = torch.full((1, nq), cfg.T, dtype=torch.int64)
    Q = make_queries(cfg, 7, inp["mu"], inp["topic"], qp, dev).contiguous()
    qp = qp.to(dev)
    layout = lsa.make_layout(cfg.d, cfg.H_kv, cfg.H_q, G["K"].dtype, tree)
    cache = lsa.LsaCache(cache_buf, layout, 1, cfg.T, cfg.T)
    lr = torch.empty(1, nq, cfg.H_kv, cfg.k, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, nq, cfg.H_kv, dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    search = "tree" if tree else "flat"
    newK = G["K"][:, :, cfg.T].clone()
    newV = G["V"][:, :, cfg.T].clone()
    rows = kv_rows(G["K"], cfg.T)
    scfg = lsa.select_cfg(cfg.k, cfg.n_sinks, cfg.window, search, cfg.beam)
    wsel = torch.empty(lsa.select_workspace_bytes(cache, scfg, nq, cfg.H_q), dtype=torch.uint8, device=dev)
    wat = torch.empty(max(1, lsa.attend_workspace_bytes(Q, cfg.H_kv, cfg.k, cfg.window)), dtype=torch.uint8,
                      device=dev)

    def step():
        append_kv(G, rows, newK, newV)
        lsa.select(Q, cache, qp, G["W"], cfg.k, cfg.n_sinks, cfg.window, search=search, beam=cfg.beam, out=(lr, cnt),
                   workspace=wsel)
        lsa.sparse_attend(Q, G["K"], G["V"], qp, lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window, O=O, workspace=wat)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    ms = graph_replay_ms(step, (lr, cnt, O), 20)
    # algorithmic bytes of a step: per (query, KV head), the centroids of every scored tree level (the
    # children of the beam, where they outnumber it) and the gathered key and value rows
    units = nq * cfg.H_kv
    info = cache.info()
    node_reads = 0
    if tree:
        sizes = [info.level_size[lev] for lev in range(info.n_levels)]
        for lev in range(info.n_levels - 1):
            cand = min(2 * cfg.beam, sizes[lev])
            node_reads += cand if cand > cfg.beam else 0
    rows = float(cnt.clamp_min(0).float().mean()) + cfg.window + cfg.n_sinks
    alg = units * (node_reads * 64 * 2 + rows * 2 * cfg.d * 2)
    return dict(queries_per_s=nq / (ms / 1e3), ms_per_step=ms, timing="hip graph replay", batch=nq, search=search,
                beam=cfg.beam, mean_lr=float(cnt.float().mean()), alg_bytes_per_step=alg,
                hbm_frac=(alg / (ms / 1e3) / 1e9) / HBM_PEAK_GBS)


def run_crossover(args):
    """Flat vs tree decode on one shared cache as the context grows (the
    pages' claim: the tree pays off only for long contexts with many
    concurrent decodes).  For each T, one sequence of the 10M-layer recipe
    (16,384 topics, 8 / 40 heads, d = 128, k = 2048, beam 64) is bucketed
    with its tree; for each batch B, B decode queries at position T (query
    recipe of the prefill) run one step — K/V append, select, attend — as a
    HIP-graph replay, with flat search (every visible bucket scored) and with
    tree search.  Prints one JSON line per (T, B, search)."""
    from synth.topics import make_queries
    dev = torch.device("cuda:0")
    out = []
    for T in args.cross_T:
        cfg = get_config(5, T=T)
        log(f"crossover: generating T={T}")
        inp = layer_inputs(cfg, seed=0, device=dev, T_cap=T + 1, queries=False)
        g = torch.Generator(device=dev)
        g.manual_seed(12345)
        kn = torch.randn(cfg.B, cfg.H_kv, cfg.d, generator=g, device=dev)
        inp["K"][:, :, T] = (kn / kn.norm(dim=-1, keepdim=True)).to(inp["K"].dtype)
        inp["V"][:, :, T] = torch.randn(cfg.B, cfg.H_kv, cfg.d, generator=g, device=dev).to(inp["V"].dtype)
        G = {k: inp[k] for k in ("K", "V", "W")}
        cache = lsa.build_buckets(G["K"], G["W"], T=T, n_q_heads=cfg.H_q, build_tree=True)
        newK = G["K"][:, :, T].clone()
        newV = G["V"][:, :, T].clone()
        rows = kv_rows(G["K"], T)
        for B in args.cross_B:
            qp = torch.full((1, B), T, dtype=torch.int64)
            Q = make_queries(cfg, 7, inp["mu"], inp["topic"], qp, dev).contiguous()
            qp = qp.to(dev)
            lr = torch.empty(1, B, cfg.H_kv, cfg.k, dtype=torch.int32, device=dev)
            cnt = torch.empty(1, B, cfg.H_kv, dtype=torch.int32, device=dev)
            O = torch.empty_like(Q)
            wat = torch.empty(max(1, lsa.attend_workspace_bytes(Q, cfg.H_kv, cfg.k, cfg.window)), dtype=torch.uint8,
                              device=dev)
            for search in ("flat", "tree"):
                scfg = lsa.select_cfg(cfg.k, cfg.n_sinks, cfg.window, search, cfg.beam)
                wsel = torch.empty(lsa.select_workspace_bytes(cache, scfg, B, cfg.H_q), dtype=torch.uint8, device=dev)

                def step():
                    append_kv(G, rows, newK, newV)
                    lsa.select(Q, cache, qp, G["W"], cfg.k, cfg.n_sinks, cfg.window, search=search, beam=cfg.beam,
                               out=(lr, cnt), workspace=wsel)
                    lsa.sparse_attend(Q, G["K"], G["V"], qp, lr, cnt, T, cfg.k, cfg.n_sinks, cfg.window, O=O,
                                      workspace=wat)

                for _ in range(3):
                    step()
                torch.cuda.synchronize()
                ms = graph_replay_ms(step, (lr, cnt, O), 20)
                rec = dict(study="decode crossover", T=T, batch=B, search=search, beam=cfg.beam if search == "tree" else 0,
                           ms_per_step=ms, queries_per_s=B / (ms / 1e3), mean_lr=float(cnt.float().mean()))
                out.append(rec)
                print(json.dumps(rec), flush=True)
        del inp, G, cache, newK, newV
        torch.cuda.empty_cache()
    return out


def graph_replay_ms(step, outs, n):
    """Capture one decode step into a HIP graph, check that replays reproduce
    the eager step's outputs exactly (with eager work and synchronisations in
    between), and return the mean time of n back-to-back replays in ms."""
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay differs from the eager decode step")
        step()
        torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n


def run_decode(args):
    cfg = get_config(3)
    dev = torch.device("cuda:0")
    log("generating decode-16x1m on the GPU")
    inp = decode_inputs(cfg, seed=0, device=dev)
    G = {k: inp[k].contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    del inp["K"], inp["V"]
    KV = pair_kv(G)
    cache = lsa.build_buckets(G["K"], G["W"], T=cfg.T, n_q_heads=cfg.H_q)
    rows = kv_rows(G["K"], cfg.T)
    rows2 = torch.cat([rows, rows + G["K"].numel() // G["K"].shape[-1]])
    newKV = torch.cat([G["K"][:, :, cfg.T].reshape(-1, cfg.d), G["V"][:, :, cfg.T].reshape(-1, cfg.d)])
    ws = lsa.select_workspace_bytes(cache, lsa.select_cfg(cfg.k, cfg.n_sinks, cfg.window), 1, cfg.H_q)
    wsel = torch.empty(ws, dtype=torch.uint8, device=dev)
    lr = torch.empty(cfg.B, 1, cfg.H_kv, cfg.k, dtype=torch.int32, device=dev)
    cnt = torch.empty(cfg.B, 1, cfg.H_kv, dtype=torch.int32, device=dev)
    O = torch.empty_like(G["Q"])
    wat = torch.empty(max(1, lsa.attend_workspace_bytes(G["Q"], cfg.H_kv, cfg.k, cfg.window)), dtype=torch.uint8,
                      device=dev)

    def step():
        append_kv_pair(KV, rows2, newKV)    # append the new token's key and value at row T
        lsa.select(G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, workspace=wsel,
                   out=(lr, cnt))
        lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window, O=O,
                          workspace=wat)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    n = 50
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        step()
    e.record()
    torch.cuda.synchronize()
    ms_eager = s.elapsed_time(e) / n
    ms = graph_replay_ms(step, (lr, cnt, O), n)
    # needle retrieved by every (sequence, KV head)?
    lr_c, cnt_c = lr.cpu(), cnt.cpu()
    found = sum(all(p + j in set(lr_c[b, 0, g, : cnt_c[b, 0, g]].tolist()) for j in range(4))
                for b, p in enumerate(inp["needle_pos"]) for g in range(cfg.H_kv))
    # algorithmic bytes of one step: every visible centroid once per (sequence, KV head) + gathered rows
    nl = (cfg.T // 2048) * 64
    cent_bytes = cfg.B * cfg.H_kv * nl * 64 * 2
    gather = cfg.B * cfg.H_kv * (int(cnt_c.clamp_min(0).sum()) / (cfg.B * cfg.H_kv) + cfg.window + cfg.n_sinks) * 512
    alg = cent_bytes + gather
    # streaming growth: a block of 2048 new tokens per sequence clustered into the cache (every 2048 steps):
    # the last block of each sequence re-added to a cache holding the ones before it
    grow = lsa.build_buckets(G["K"], G["W"], T=cfg.T - 2048, t_max=cfg.T, n_q_heads=cfg.H_q)
    grow_ms = []
    for rep in range(6):
        grow.T = cfg.T - 2048
        torch.cuda.synchronize()
        s.record()
        lsa.extend_buckets(grow, G["K"], G["W"], cfg.T)
        e.record()
        torch.cuda.synchronize()
        if rep > 0:
            grow_ms.append(s.elapsed_time(e))
    grow_block_ms = sum(grow_ms) / len(grow_ms)
    return dict(queries_per_s=cfg.B / (ms / 1e3), ms_per_step=ms, ms_per_step_eager=ms_eager, timing="hip graph replay",
                needle_found=f"{found}/{cfg.B * cfg.H_kv}",
                alg_bytes_per_step=alg, hbm_frac=(alg / (ms / 1e3) / 1e9) / HBM_PEAK_GBS,
                grow_block_ms=grow_block_ms, grow_us_per_step_amortized=grow_block_ms * 1e3 / 2048)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 4, 5],
                    help="prefill workload: 4 (1M, the default, followed by the 1M decode and the 10M layer), "
                         "5 (10M tree layer alone), or the parity configs 1 (8K fp32) and 2 (131K)")
    ap.add_argument("--attend", default="auto", choices=["auto", "gather", "bucket"],
                    help="prefill attention: per-query gather, bucket-major (each bucket's K/V read once per pass), "
                         "or auto (bucket-major when a bucket is expected in >= 2 pairs per pass)")
    ap.add_argument("--bucket-records", choices=["only", "on", "off"], default="only",
                    help="bucket-major attention takes its pairs from the selection's bucket records, the rows "
                         "with records then getting no token list (only) or getting one too (on), or takes them "
                         "from the token lists (off); the same output")
    ap.add_argument("--bm-pass", type=int, default=0,
                    help="most queries per bucket-major pass, lowered in steps of 4096 until the workspace fits "
                         "(0: 32768 where such a pass gives a bucket >= 8 pairs, else 65536)")
    ap.add_argument("--bm-mem", type=float, default=0.72,
                    help="largest share of the free device memory the bucket-major workspace may take")
    ap.add_argument("--study", choices=["crossover"], default=None,
                    help="instead of the benchmark: the flat vs tree decode crossover over --cross-T x --cross-B")
    ap.add_argument("--cross-T", type=int, nargs="+", default=[1 << 20, 1 << 21, 1 << 22, 1 << 23, 10485760])
    ap.add_argument("--cross-B", type=int, nargs="+", default=[1, 4, 16, 64])
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-10m", action="store_true", help="skip the 10M-token tree layer of the default run")
    ap.add_argument("--steps-10m", type=int, default=2, help="timed steps of the 10M layer (about 8 s each)")
    ap.add_argument("--warmup-10m", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run one plain 1 GiB device copy (a known-size kernel for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the LSA path here has no multi-GPU sharding); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.study == "crossover":
        run_crossover(args)
        return
    if args.calibrate:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)            # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    res, cfg, inp = run_prefill(args, args.config, args.steps, args.warmup)
    log(f"prefill {res['value']:.0f} tokens/s, {res['ms_per_step']:.1f} ms/step")
    del inp
    torch.cuda.empty_cache()
    if not args.no_decode and args.config == 4:
        try:
            res["decode_1m"] = run_decode(args)
            log(f"decode {res['decode_1m']}")
        except torch.cuda.OutOfMemoryError as exc:  # pragma: no cover
            res["decode_1m"] = {"error": str(exc)[:200]}
        torch.cuda.empty_cache()
    if not args.no_10m and args.config == 4:
        # the metric's second prefill context: the 10M-token tree layer, with a fixed small step count
        r10, _, inp10 = run_prefill(args, 5, args.steps_10m, args.warmup_10m)
        del inp10
        torch.cuda.empty_cache()
        res["prefill_10m"] = {k: r10[k] for k in ("value", "unit", "steps", "warmup", "ms_per_step", "config",
                                                   "breakdown_ms", "roofline", "bucket_major_fallbacks",
                                                   "decode_shared") if k in r10}
        log(f"prefill 10M {r10['value']:.0f} tokens/s, {r10['ms_per_step']:.1f} ms/step")
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cfg_cpu = get_config(args.config)
        small = cfg_cpu.scaled(T=min(cfg_cpu.T, 64 * 2048))
        inp_cpu = layer_inputs(small, seed=0)
        res["cpu_baseline"] = cpu_baseline(cfg_cpu, inp_cpu)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
