"""Parity of the training-free projection (lsa_pca_projection: the 64 leading
principal directions of the keys) with the oracle, and the whole path run on
such a projection."""

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_indexing_latent_amd as lsa
from synth import get_config, layer_inputs
from tests.parity import MARGIN, compare_ward, gpu_partitions, lr_row

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _rows(K):
    """every key row of K [B, H_kv, T, d] as float64 [N, d]"""
    return K.double().reshape(-1, K.shape[-1]).cpu().numpy()


def _check(K, W_gpu, ev_gpu, strict_sub):
    X = _rows(K)
    W_o, lam = O.pca_projection(X, 64)
    Wg = W_gpu.double().cpu().numpy()
    C = np.cov(X.T, bias=True)
    d = X.shape[1]
    # eigenvalues (fp32 Jacobi on an fp32/fp64-accumulated covariance)
    assert np.max(np.abs(ev_gpu.double().cpu().numpy() - lam)) <= 1e-4 * lam[0], "eigenvalues"
    # orthonormal columns (bf16 storage rounds each entry to 2^-9 relative; in fp32 each column has been
    # through ~10^3 rotations of ~6e-8 relative error each)
    ortho = 2e-2 if W_gpu.dtype == torch.bfloat16 else 1e-4
    assert np.max(np.abs(Wg.T @ Wg - np.eye(64))) <= ortho, "orthonormality"
    # captured variance: as much as the leading 64 eigenvalues hold
    cap = np.trace(Wg.T @ C @ Wg) / np.trace(Wg.T @ Wg) * 64
    assert cap >= (1 - 2e-3) * lam[:64].sum(), "captured variance"
    # the spanned subspace, where the eigen-gap makes it well defined (Davis-Kahan: error ~ noise / gap)
    gap = (lam[63] - lam[64]) if d > 64 else lam[0]
    Qg, _ = np.linalg.qr(Wg)
    dist = np.linalg.norm(Qg @ Qg.T - W_o @ W_o.T, 2)
    bound = (2e-2 if W_gpu.dtype == torch.bfloat16 else 1e-4) + 1e-5 * lam[0] / max(gap, 1e-30)
    print(f"[pca] d={d} {W_gpu.dtype}: gap/lam1 {gap / lam[0]:.2e}, subspace distance {dist:.2e} (bound {bound:.2e})",
          flush=True)
    if strict_sub:
        assert dist <= bound, "subspace"
    return W_o


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pca_designed_spectrum(dtype):
    """Keys with a clear gap after the 64th direction: the subspace must match closely."""
    g = torch.Generator().manual_seed(11)
    d, T = 128, 6000
    R, _ = torch.linalg.qr(torch.randn(d, d, generator=g, dtype=torch.float64))
    sig = torch.cat([torch.linspace(3.0, 1.0, 64), torch.linspace(0.3, 0.05, 64)]).double()
    X = (torch.randn(2 * T, d, generator=g, dtype=torch.float64) * sig) @ R.T + 0.1
    K = X.reshape(1, 2, T, d).to(dtype).contiguous()
    W, ev = lsa.pca_projection(K.to(DEV), with_eigvals=True)
    torch.cuda.synchronize()
    _check(K, W, ev, strict_sub=True)


def test_pca_fp32_d64_full_basis():
    cfg = get_config(1, T=8192)
    inp = layer_inputs(cfg, seed=5, queries=False)
    W, ev = lsa.pca_projection(inp["K"].to(DEV).contiguous(), with_eigvals=True)
    torch.cuda.synchronize()
    _check(inp["K"], W, ev, strict_sub=True)


def test_pca_bf16_topic_keys_and_path():
    """On the 131k-layer recipe (topic-mixture keys, d = 128): eigenvalues, orthonormality and captured
    variance against the oracle; then the whole path (build, flat select) run on the GPU's projection
    matches the oracle run on the same projection."""
    cfg = get_config(2, T=16384, H_kv=2, H_q=10, n_topics=64)
    inp = layer_inputs(cfg, seed=6)
    Kd = inp["K"].to(DEV).contiguous()
    W, ev = lsa.pca_projection(Kd, with_eigvals=True)
    torch.cuda.synchronize()
    _check(inp["K"], W, ev, strict_sub=False)
    G = {k: inp[k].to(DEV).contiguous() for k in ("Q", "q_pos")}
    cache = lsa.build_buckets(Kd, W, n_q_heads=cfg.H_q)
    lr, cnt = lsa.select(G["Q"], cache, G["q_pos"], W, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    lr, cnt = lr.cpu().numpy(), cnt.cpu().numpy()
    Wn = W.double().cpu().numpy()
    rng = np.random.default_rng(3)
    res = dict(exact=0, excused=0, unexcused=0)
    for g in range(cfg.H_kv):
        # Ward on the GPU's projection: every block against the oracle's own Ward (margin protocol); the
        # selections are then judged on the oracle's cache over those (verified) partitions, by the
        # selection margin alone
        Kg = inp["K"][0, g].double().numpy()
        own = O.build_head_cache(Kg, Wn, "bf16", processes=8)
        gp = gpu_partitions(cache, 0, g)
        ward = compare_ward(own["entries"], own["clusters"], gp)
        print(f"[pca] g={g} ward {ward['exact']}/{ward['blocks']} exact, {ward['excused']} excused", flush=True)
        assert ward["unexcused"] == 0
        oc = O.build_head_cache(Kg, Wn, "bf16", clusters=gp)
        for t in rng.integers(2048, cfg.T, 60):
            qh = O.query_latent(inp["Q"][0, t, g * cfg.G:(g + 1) * cfg.G].double().numpy(), Wn, "bf16")
            ref, info = O.select_flat(qh, oc, int(t), cfg.k, cfg.n_sinks, cfg.window, with_margin=True)
            if np.array_equal(ref, lr_row(lr[0, t, g], cnt[0, t, g])):
                res["exact"] += 1
            else:
                res["excused" if info["margin"] < MARGIN else "unexcused"] += 1
    print(f"[pca] path on the PCA projection: selections {res}", flush=True)
    assert res["unexcused"] == 0 and res["exact"] >= 100
