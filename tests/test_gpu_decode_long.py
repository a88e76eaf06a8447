"""Decode selection past 1M tokens, where the materialized scan writes exact bf16 scores instead of int8 bounds
(more than 2048 tiles of 16 buckets per (sequence, KV head)): its lists must equal the fused strategy's bit for
bit (the same scores, ranked by the same rule; the fused strategy is checked against the oracle elsewhere)."""

import pytest
import torch

import sparse_attention_indexing_latent_amd as lsa
from synth import get_config, layer_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_decode_past_1m_exact_scan_equals_fused():
    T = 1030 * 2048                      # 4120 tiles per (sequence, KV head)
    cfg = get_config(2, T=T, B=2, H_kv=2, H_q=10, n_topics=2048, k=2048, window=1024)
    qp = torch.full((cfg.B, 1), T, dtype=torch.int64)
    print("[decode-long] generating", flush=True)
    inp = layer_inputs(cfg, seed=5, device=DEV, T_cap=T + 1, q_positions=qp)
    G = {k: inp[k].contiguous() for k in ("K", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], T=T, n_q_heads=cfg.H_q)
    args = (G["Q"], cache, G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window)
    lr_m, cnt_m = lsa.select(*args, strategy="materialized")
    lr_f, cnt_f = lsa.select(*args, strategy="fused")
    torch.cuda.synchronize()
    assert torch.equal(cnt_m, cnt_f)
    for b in range(cfg.B):
        for g in range(cfg.H_kv):
            n = int(cnt_m[b, 0, g])
            assert n == cfg.k
            assert torch.equal(lr_m[b, 0, g, :n], lr_f[b, 0, g, :n])
    print(f"[decode-long] materialized == fused on {cfg.B * cfg.H_kv} units at T = {T}", flush=True)
