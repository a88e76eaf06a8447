"""Topic-mixture workload generator.

The pages describe keys that are semantically clustered and arrive in runs of
adjacent tokens sharing a subject (zhichai.net explainer, ch.2 "semantic
clustering": pooling adjacent keys is justified by topical locality), and
queries that look for an earlier subject.  No public dataset is available here,
so every workload is synthesised from a seed:

* topic directions mu[g, j]: i.i.d. Gaussian, normalised, one set per KV head;
* runs of 16..256 tokens (uniform), each with a uniform random topic, shared by
  all KV heads, the last run cut at T;
* keys K[g, t] = normalise(mu[g, topic(t)] + eps / sqrt(kappa)), eps ~ N(0, I_d),
  kappa = 20 (a von Mises-Fisher-like cloud on the sphere), cast to the dtype;
* values V ~ N(0, 1);
* projection W ~ N(0, 1) / sqrt(d), shape [d, 64];
* the query at position t picks s uniform in [0, t-1] (s = 0 at t = 0) and, for
  every query head h of KV group g, Q[t, h] = alpha * normalise(mu[g, topic(s)]
  + eps_h / sqrt(kappa)) with alpha = 8 sqrt(d), so logits are 8 * cosine;
* the decode workload plants a needle: one pooled entry (4 keys) of each KV
  head set to a fresh unit direction nu[g], and the new query aims at nu[g].

Every tensor is drawn from its own torch.Generator whose seed is a hash of
(seed, config, tensor name, indices), so a slice is reproducible on its own.
The generator normalises vectors to build inputs; it performs none of the
method's steps (no latent projection, pooling, clustering, scoring or
attention).
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import numpy as np
import torch

KAPPA = 20.0


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One benchmark/parity workload (shapes, dtype, selection parameters)."""

    cid: int
    name: str
    T: int                  # tokens in the K/V cache (prefill length or decode context)
    H_kv: int
    H_q: int
    d: int
    dtype: str              # "f32" or "bf16"
    n_topics: int
    k: int                  # long-range token budget
    n_sinks: int
    window: int
    search: str             # "flat" or "tree"
    beam: int = 0           # tree beam width
    B: int = 1              # independent sequences
    decode: bool = False    # one new query per sequence at position T
    needle: bool = False
    decode_batch: int = 0   # cfg5: decode queries on the shared cache

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    def scaled(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads, in order: a tiny fp32 layer; prefill at 131,072 tokens;
# a 16-sequence decode step at 1M context; prefill at 1M; prefill at 10M with
# the tree search (beam = k / (4 * 8) leaves) plus an 8-query decode step.
WORKLOADS = {
    1: LayerConfig(1, "tiny-f32-8k", 8192, 1, 4, 64, "f32", 32, 256, 4, 128, "flat"),
    2: LayerConfig(2, "prefill-131k", 131072, 8, 40, 128, "bf16", 512, 2048, 4, 1024, "flat"),
    3: LayerConfig(3, "decode-16x1m", 1048576, 8, 40, 128, "bf16", 4096, 2048, 4, 1024, "flat",
                   B=16, decode=True, needle=True),
    4: LayerConfig(4, "prefill-1m", 1048576, 8, 40, 128, "bf16", 4096, 2048, 4, 1024, "flat"),
    5: LayerConfig(5, "prefill-10m", 10485760, 8, 40, 128, "bf16", 16384, 2048, 4, 1024, "tree",
                   beam=64, decode_batch=8),
}


def get_config(cid: int, **overrides) -> LayerConfig:
    cfg = WORKLOADS[cid]
    return cfg.scaled(**overrides) if overrides else cfg


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(device, *key) -> torch.Generator:
    digest = hashlib.sha256(repr(key).encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(digest[:8], "little") & ((1 << 63) - 1))
    return g


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def topic_directions(cfg: LayerConfig, seed: int, b: int, device) -> torch.Tensor:
    """[H_kv, n_topics, d] fp32 unit vectors (per sequence b, per KV head)."""
    out = torch.empty(cfg.H_kv, cfg.n_topics, cfg.d, dtype=torch.float32, device=device)
    for g in range(cfg.H_kv):
        gen = _gen(device, seed, cfg.cid, "topics", b, g)
        out[g] = _unit(torch.randn(cfg.n_topics, cfg.d, generator=gen, device=device))
    return out


def topic_runs(cfg: LayerConfig, seed: int, b: int, T: int) -> torch.Tensor:
    """int64 [T] topic id of every token (runs of 16..256 tokens), built on CPU."""
    gen = _gen("cpu", seed, cfg.cid, "runs", b)
    n_max = T // 16 + 2
    lengths = torch.randint(16, 257, (n_max,), generator=gen)
    topics = torch.randint(0, cfg.n_topics, (n_max,), generator=gen)
    csum = torch.cumsum(lengths, 0)
    n_runs = int(torch.searchsorted(csum, torch.tensor(T)).item()) + 1
    return torch.repeat_interleave(topics[:n_runs], lengths[:n_runs])[:T].contiguous()


def _keys_for(cfg, seed, b, g, mu_g, topic_of, t0, t1, device, dt):
    gen = _gen(device, seed, cfg.cid, "keynoise", b, g, t0)
    eps = torch.randn(t1 - t0, cfg.d, generator=gen, device=device)
    return _unit(mu_g[topic_of[t0:t1]] + eps / math.sqrt(KAPPA)).to(dt)


CHUNK = 1 << 20


def layer_inputs(cfg: LayerConfig, seed: int = 0, device="cpu", *, T_cap: Optional[int] = None,
                 queries: bool = True, q_positions: Optional[torch.Tensor] = None):
    """Keys, values, projection and (optionally) queries of one prefill layer.

    Returns a dict with
      K, V : [B, H_kv, T_cap, d] (config dtype), rows >= T are zero
      W    : [d, 64] (config dtype)
      Q    : [B, n_q, H_q, d] for positions q_pos (default: all 0..T-1)
      q_pos: int64 [B, n_q]
      topic: int64 [B, T] topic of every token (CPU)
    """
    dev = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    T = cfg.T
    T_cap = T if T_cap is None else T_cap
    K = torch.zeros(cfg.B, cfg.H_kv, T_cap, cfg.d, dtype=dt, device=dev)
    V = torch.zeros_like(K)
    topics_all = []
    mus = []
    for b in range(cfg.B):
        mu = topic_directions(cfg, seed, b, dev)
        mus.append(mu)
        topic_of = topic_runs(cfg, seed, b, T)
        topics_all.append(topic_of)
        topic_dev = topic_of.to(dev)
        for g in range(cfg.H_kv):
            for t0 in range(0, T, CHUNK):
                t1 = min(T, t0 + CHUNK)
                K[b, g, t0:t1] = _keys_for(cfg, seed, b, g, mu[g], topic_dev, t0, t1, dev, dt)
                gen = _gen(dev, seed, cfg.cid, "values", b, g, t0)
                V[b, g, t0:t1] = torch.randn(t1 - t0, cfg.d, generator=gen, device=dev).to(dt)
    gen = _gen(dev, seed, cfg.cid, "W")
    W = (torch.randn(cfg.d, 64, generator=gen, device=dev) / math.sqrt(cfg.d)).to(dt)
    out = dict(K=K, V=V, W=W, topic=torch.stack(topics_all), mu=torch.stack(mus))
    if queries:
        if q_positions is None:
            q_positions = torch.arange(T, dtype=torch.int64).unsqueeze(0).repeat(cfg.B, 1)
        out["q_pos"] = q_positions.to(dev)
        out["Q"] = make_queries(cfg, seed, out["mu"], out["topic"], q_positions, dev)
    return out


def make_queries(cfg: LayerConfig, seed: int, mu: torch.Tensor, topic: torch.Tensor,
                 q_pos: torch.Tensor, device) -> torch.Tensor:
    """Q [B, n_q, H_q, d]: each query aims at the topic of a random earlier token."""
    dev = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    B, n_q = q_pos.shape
    Q = torch.empty(B, n_q, cfg.H_q, cfg.d, dtype=dt, device=dev)
    alpha = 8.0 * math.sqrt(cfg.d)
    qc = 1 << 16
    for b in range(B):
        pos_cpu = q_pos[b].cpu()
        for i0 in range(0, n_q, qc):
            i1 = min(n_q, i0 + qc)
            pos = pos_cpu[i0:i1]
            gen_c = _gen("cpu", seed, cfg.cid, "qpick", b, i0)
            u = torch.rand(i1 - i0, generator=gen_c, dtype=torch.float64)
            src = torch.clamp((u * pos.to(torch.float64)).floor().to(torch.int64), min=0)
            src = torch.minimum(src, torch.clamp(pos - 1, min=0))
            src = torch.clamp(src, max=topic.shape[1] - 1)
            tau = topic[b][src].to(dev)
            gen = _gen(dev, seed, cfg.cid, "qnoise", b, i0)
            eps = torch.randn(i1 - i0, cfg.H_q, cfg.d, generator=gen, device=dev)
            centre = mu[b][:, tau, :].repeat_interleave(cfg.G, dim=0).transpose(0, 1)  # [n, H_q, d]
            Q[b, i0:i1] = (alpha * _unit(centre + eps / math.sqrt(KAPPA))).to(dt)
    return Q


def decode_inputs(cfg: LayerConfig, seed: int = 0, device="cpu"):
    """Decode step: B sequences with T cached tokens plus the new token at T.

    K/V hold T+1 rows per sequence (row T is the appended token).  With
    cfg.needle, one pooled entry per KV head (positions p..p+3, p = 0 mod 4,
    p in [4, T - window - 4)) is set to a fresh unit direction nu[g] and the
    new query of every head in group g aims at nu[g].  Without a needle
    (cfg.decode_batch > 0) the decode queries come from the prefill query
    recipe, all at position T on sequence 0.
    """
    dev = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    T = cfg.T
    inp = layer_inputs(cfg, seed, dev, T_cap=T + 1, queries=False)
    K, V, mu = inp["K"], inp["V"], inp["mu"]
    alpha = 8.0 * math.sqrt(cfg.d)
    needle_pos = []
    if cfg.needle:
        Q = torch.empty(cfg.B, 1, cfg.H_q, cfg.d, dtype=dt, device=dev)
        for b in range(cfg.B):
            gen_c = _gen("cpu", seed, cfg.cid, "needlepos", b)
            p = 4 * int(torch.randint(1, (T - cfg.window - 4) // 4, (1,), generator=gen_c).item())
            needle_pos.append(p)
            gen = _gen(dev, seed, cfg.cid, "needle", b)
            nu = _unit(torch.randn(cfg.H_kv, cfg.d, generator=gen, device=dev))
            K[b, :, p:p + 4, :] = nu.to(dt).unsqueeze(1)
            gen = _gen(dev, seed, cfg.cid, "needleq", b)
            eps = torch.randn(cfg.H_q, cfg.d, generator=gen, device=dev)
            Q[b, 0] = (alpha * _unit(nu.repeat_interleave(cfg.G, 0) + eps / math.sqrt(KAPPA))).to(dt)
        q_pos = torch.full((cfg.B, 1), T, dtype=torch.int64)
    else:
        nq = max(1, cfg.decode_batch)
        q_pos = torch.full((cfg.B, nq), T, dtype=torch.int64)
        Q = make_queries(cfg, seed, mu, inp["topic"], q_pos, dev)
    # the appended token: a random-topic key and a Gaussian value
    for b in range(cfg.B):
        gen = _gen(dev, seed, cfg.cid, "newtok", b)
        tp = torch.randint(0, cfg.n_topics, (1,), generator=gen, device=dev)
        eps = torch.randn(cfg.H_kv, cfg.d, generator=gen, device=dev)
        K[b, :, T, :] = _unit(mu[b][:, tp[0], :] + eps / math.sqrt(KAPPA)).to(dt)
        V[b, :, T, :] = torch.randn(cfg.H_kv, cfg.d, generator=gen, device=dev).to(dt)
    return dict(K=K, V=V, W=inp["W"], Q=Q, q_pos=q_pos.to(dev), topic=inp["topic"], mu=mu,
                needle_pos=needle_pos)


def random_lr_lists(cfg: LayerConfig, q_pos: torch.Tensor, seed: int = 0, n_blocks: Optional[int] = None,
                    fill: float = 1.0):
    """Synthetic long-range index lists for testing the attention call alone.

    For each (b, query, KV head) draws up to k distinct sorted token indices from
    [min(n_sinks, t+1), l0) where l0 is the start of the local window widened to
    the query's own unbucketed block; returns (lr_idx int32 [B, n_q, H_kv, k]
    padded with -1, lr_cnt int32 [B, n_q, H_kv]).  CPU tensors.
    """
    B, n_q = q_pos.shape
    k = cfg.k
    idx = torch.full((B, n_q, cfg.H_kv, max(k, 1)), -1, dtype=torch.int32)
    cnt = torch.zeros(B, n_q, cfg.H_kv, dtype=torch.int32)
    nb_all = cfg.T // 2048 if n_blocks is None else n_blocks
    digest = hashlib.sha256(repr((seed, cfg.cid, "randlr")).encode()).digest()
    rng = np.random.default_rng(int.from_bytes(digest[:8], "little"))
    idx_np = idx.numpy()
    cnt_np = cnt.numpy()
    for b in range(B):
        for i in range(n_q):
            t = int(q_pos[b, i])
            nvis = min(t // 2048, nb_all)
            l0 = max(0, min(t - cfg.window + 1, 2048 * nvis))
            lo = min(cfg.n_sinks, t + 1)
            span = max(0, l0 - lo)
            for g in range(cfg.H_kv):
                want = min(k, int(span * fill))
                if want <= 0:
                    continue
                pick = np.sort(rng.choice(span, size=want, replace=False)) + lo
                idx_np[b, i, g, :want] = pick
                cnt_np[b, i, g] = want
    return idx[..., :k] if k > 0 else idx[..., :0], cnt
