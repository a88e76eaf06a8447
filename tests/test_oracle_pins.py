"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test names what fixes the expected value: brute force, a library
routine (SciPy's Ward linkage, torch's scaled-dot-product attention, torch's
bf16 cast), a closed form, or a hand-checkable case.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from tests.bruteforce_ward import brute_ward

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _canon(clusters):
    return sorted(tuple(sorted(c)) for c in clusters)


# ---------------------------------------------------------------- rounding

def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x32 = (rng.standard_normal(20000) * rng.choice([1e-3, 0.1, 1, 30], 20000)).astype(np.float32)
    ours = O.round_to(x32.astype(np.float64), "bf16")
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_round_bf16_half_even_cases():
    # 1 + 2^-8 is half way between 1 and 1 + 2^-7: ties go to the even 1.0
    assert O.round_to(np.array([1 + 2 ** -8]), "bf16")[0] == 1.0
    assert O.round_to(np.array([1 + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6
    assert O.round_to(np.array([-(1 + 2 ** -8)]), "bf16")[0] == -1.0
    assert O.round_to(np.array([0.0]), "bf16")[0] == 0.0


def test_round_f32_is_ieee_cast():
    x = np.array([1 + 2 ** -24, 1 + 3 * 2 ** -24, 0.1])
    r = O.round_to(x, "f32")
    assert r[0] == 1.0 and r[1] == 1 + 2 ** -22 and r[2] == np.float32(0.1)


# ---------------------------------------------------------------- latents and pooling

def test_latents_unit_norm_and_identity_projection():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((64, 64))
    u = O.key_latents(K, np.eye(64) * 3.7)          # scale of W cancels
    assert np.allclose(np.linalg.norm(u, axis=1), 1.0, atol=1e-12)
    assert np.allclose(u, K / np.linalg.norm(K, axis=1, keepdims=True), atol=1e-12)


def test_zero_key_gives_zero_latent():
    u = O.key_latents(np.zeros((4, 8)), np.ones((8, 64)))
    assert np.all(u == 0)


# ---------------------------------------------------------------- query latent

def _exact_unit_rows():
    """Integer query rows whose squared norm is exactly 1024^2, so q / ||q|| is
    exact in float64; with the identity projection the latent is q / 1024.
    Row 0: 514/1024 = 0.5 + 2^-9 sits half way between the bf16 values 0.5 and
    0.50390625 (spacing 2^-8 in [0.5, 1)); ties go to the even 0.5.  Row 1:
    518/1024 sits half way between 0.50390625 (odd last bit) and 0.5078125
    (even): it rounds up.  885/1024 and 883/1024 lie 1/4 and 3/4 of a step
    above 0.86328125 = 884/1024 and round to it.  The small components are
    exact in bf16."""
    q = np.zeros((2, 64))
    q[0, :6] = [514, 885, 33, 8, 1, 1]
    q[1, :5] = [518, 883, 23, 5, 3]
    assert np.all((q * q).sum(axis=1) == 1024 ** 2)
    want = np.zeros((2, 64))
    want[0, :6] = [0.5, 0.86328125, 33 / 1024, 8 / 1024, 1 / 1024, 1 / 1024]
    want[1, :5] = [0.5078125, 0.86328125, 23 / 1024, 5 / 1024, 3 / 1024]
    return q, want


def test_query_latent_normalises_then_rounds_half_even():
    q, want = _exact_unit_rows()
    got = O.query_latent(q, np.eye(64), "bf16")
    assert np.array_equal(got, want)
    # without the rounding the half-way components would be kept exactly
    exact = O.query_latent(q, np.eye(64), "f64")
    assert exact[0, 0] == 514 / 1024 and exact[1, 0] == 518 / 1024
    # fp32 storage keeps all of them (every component is a multiple of 2^-10)
    assert np.array_equal(O.query_latent(q, np.eye(64), "f32"), q / 1024)


def test_query_latent_scale_invariant_and_projected():
    q, want = _exact_unit_rows()
    for c in (7.5, 2.0 ** -20, 3.0e5):
        assert np.array_equal(O.query_latent(c * q, np.eye(64), "bf16"), want)
    # a projection that permutes and scales the axes: q W = 4 * (q permuted)
    perm = np.random.default_rng(3).permutation(64)
    W = np.zeros((64, 64))
    W[np.arange(64), perm] = 4.0
    got = O.query_latent(q, W, "bf16")
    assert np.array_equal(got[:, perm], want)
    # a head dimension larger than the latent: W [128, 64] reading only the first 64 dims
    q2 = np.concatenate([q, np.full((2, 64), 0.0)], axis=1)
    W2 = np.concatenate([np.eye(64), np.full((64, 64), 9.0)], axis=0)
    assert np.array_equal(O.query_latent(q2, W2, "bf16"), want)
    # the unit norm holds before rounding, and a zero query stays zero
    assert np.allclose(np.linalg.norm(O.query_latent(q, np.eye(64), "f64"), axis=1), 1.0, atol=0)
    assert np.all(O.query_latent(np.zeros((1, 64)), np.eye(64), "bf16") == 0)


def test_pooling_is_mean_of_four():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((4 * 5 + 3, 64))
    e = O.pooled_entries(u)
    assert e.shape == (5, 64)
    row = rng.standard_normal(64)
    same = O.pooled_entries(np.tile(row, (4, 1)))
    assert np.allclose(same[0], row)
    assert np.allclose(e[2], (u[8] + u[9] + u[10] + u[11]) / 4)


# ---------------------------------------------------------------- Ward

@pytest.mark.parametrize("cap", [2, 3, 4, 16])
@pytest.mark.parametrize("seed", range(6))
def test_ward_matches_bruteforce(cap, seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(5, 13))
    E = rng.standard_normal((n, 6))
    for target in range(1, n + 1):
        if (n + cap - 1) // cap > target:      # infeasible under the cap
            continue
        ours = O.ward_block(E, cap=cap, target=target)["clusters"]
        ref = brute_ward(E, cap, target)
        assert _canon(ours) == _canon(ref), (cap, seed, target)


def test_ward_matches_scipy_when_cap_does_not_bind():
    from scipy.cluster.hierarchy import fcluster, linkage
    for seed in range(10):
        rng = np.random.default_rng(seed)
        n = 16
        E = rng.standard_normal((n, 8))
        ours = O.ward_block(E, cap=16, mean_bucket=8, margins=True)
        Z = linkage(E, method="ward")
        lab = fcluster(Z, t=2, criterion="maxclust")
        ref = [list(np.flatnonzero(lab == v)) for v in np.unique(lab)]
        assert _canon(ours["clusters"]) == _canon(ref)


def test_ward_full_block_matches_scipy_without_cap():
    from scipy.cluster.hierarchy import fcluster, linkage
    rng = np.random.default_rng(7)
    E = rng.standard_normal((512, 64)) * 0.1 + rng.standard_normal((1, 64))
    ours = O.ward_block(E, cap=512, target=64, margins=True)
    Z = linkage(E, method="ward")
    lab = fcluster(Z, t=64, criterion="maxclust")
    ref = [list(np.flatnonzero(lab == v)) for v in np.unique(lab)]
    assert _canon(ours["clusters"]) == _canon(ref)


def test_ward_invariants_on_topic_block():
    # a pooled block from the topic-mixture generator
    from synth import get_config, layer_inputs
    cfg = get_config(2, T=2048, H_kv=1, H_q=5, n_topics=8)
    inp = layer_inputs(cfg, seed=3, queries=False)
    K = inp["K"][0, 0].double().numpy()
    W = inp["W"].double().numpy()
    e = O.pooled_entries(O.key_latents(K, W))
    res = O.ward_block(e, margins=True)
    sizes = [len(c) for c in res["clusters"]]
    assert len(sizes) == 64 and sum(sizes) == 512
    assert max(sizes) <= 16 and min(sizes) >= 1
    h = np.array(res["heights"])
    assert np.all(np.diff(h) >= -1e-12 * np.maximum(1.0, h[1:]))
    assert sorted(i for c in res["clusters"] for i in c) == list(range(512))
    # ids are ordered and each cluster's id is its smallest member
    ids = [c[0] for c in res["clusters"]]
    assert ids == sorted(ids)


def test_ward_feasible_for_all_sizes():
    rng = np.random.default_rng(5)
    for n in [1, 2, 7, 8, 9, 15, 16, 17, 100, 137]:
        E = rng.standard_normal((n, 4))
        res = O.ward_block(E)
        assert len(res["clusters"]) == -(-n // 8)
        assert max(len(c) for c in res["clusters"]) <= 16


def test_ward_tie_rule_lowest_pair():
    # four points on a square: all four edges tie; the lowest (id_A, id_B) = (0, 1) goes first
    E = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    res = O.ward_block(E, cap=16, target=3, margins=True)
    assert res["merges"][0][:2] == (0, 1)
    assert _canon(res["clusters"]) == [(0, 1), (2,), (3,)]


# ---------------------------------------------------------------- cache and tree

def _small_cache(seed=0, T=8192, tree=False, dtype="f32"):
    from synth import get_config, layer_inputs
    cfg = get_config(1, T=T)
    inp = layer_inputs(cfg, seed=seed)
    K = inp["K"][0, 0].double().numpy()
    W = inp["W"].double().numpy()
    cache = O.build_head_cache(K, W, dtype, tree=tree)
    return cfg, inp, cache


def test_centroids_unit_and_mean_of_members():
    cfg, inp, cache = _small_cache()
    assert np.allclose(np.linalg.norm(cache["cent"], axis=1), 1.0, atol=1e-6)
    # recompute from the token latents directly: mean of the member keys' unit latents
    K = inp["K"][0, 0].double().numpy()
    W = inp["W"].double().numpy()
    u = O.key_latents(K, W)
    for x in [0, 17, 100, 255]:
        tok = O.leaf_tokens(cache["members"][x])
        ref = O.normalise(u[tok].mean(axis=0, keepdims=True))[0]
        assert np.allclose(cache["cent"][x], ref, atol=1e-6)


def test_tree_root_and_depth():
    cfg, inp, cache = _small_cache(tree=True)
    levels = cache["tree"]
    NL = len(cache["sums"])
    assert NL == 256
    assert len(levels) == math.ceil(math.log2(NL)) + 1
    # root = normalised sum of every pooled entry of every full block
    root_ref = O.normalise(cache["entries"].sum(axis=0, keepdims=True))[0]
    assert np.allclose(levels[-1]["cent"][0], root_ref, atol=1e-6)
    # a level-3 node covers 8 consecutive leaves
    ref = O.normalise(cache["sums"][16:24].sum(axis=0, keepdims=True))[0]
    assert np.allclose(levels[3]["cent"][2], ref, atol=1e-6)


def test_tree_odd_counts_carry_last_node():
    sums = np.random.default_rng(3).standard_normal((5, 4))
    levels = O.build_tree(sums, "f64")
    assert [len(l["cent"]) for l in levels] == [5, 3, 2, 1]
    assert np.allclose(levels[1]["sums"][2], sums[4])
    assert np.allclose(levels[2]["sums"][1], sums[4])


# ---------------------------------------------------------------- selection

def _hand_cache():
    """One block, 64 leaves of 8 consecutive entries each; leaf x's centroid
    is a unit vector at angle x * 0.02 rad from axis 0 in the (0, 1) plane."""
    members = [np.arange(8 * x, 8 * x + 8) for x in range(64)]
    ang = 0.02 * np.arange(64)
    cent = np.zeros((64, 64))
    cent[:, 0] = np.cos(ang)
    cent[:, 1] = np.sin(ang)
    return dict(n_blocks=1, members=members, sizes=np.full(64, 8), cent=cent)


def test_select_hand_checkable():
    cache = _hand_cache()
    q = np.zeros((1, 64))
    q[0, 0] = 1.0
    t = 5000                        # block 2; block 0 visible, local = [2048*1=2048..] -> l0 = min(t-w+1, 2048)
    lr, info = O.select_flat(q, cache, t, k=40, n_sinks=4, window=128)
    # leaf 0 (score 1) holds entries 0..7 = tokens 0..31; tokens 0..3 are sinks -> 28 eligible
    # leaf 1 gives its 12 lowest tokens 32..43
    assert list(lr) == list(range(4, 32)) + list(range(32, 44))
    assert info["boundary"] == 1


def test_select_tie_goes_to_lower_id():
    cache = _hand_cache()
    cache["cent"][5] = cache["cent"][9] = np.eye(64)[2]
    q = np.zeros((1, 64))
    q[0, 2] = 1.0
    lr, info = O.select_flat(q, cache, 4096, k=32, n_sinks=0, window=1)
    assert list(lr) == list(range(5 * 32, 6 * 32))


def test_select_before_first_block_is_empty():
    cfg, inp, cache = _small_cache()
    q = np.ones((4, 64)) / 8
    for t in [0, 3, 2047]:
        lr, _ = O.select_flat(q, cache, t, 256, 4, 128)
        assert len(lr) == 0


def test_select_k_covers_everything():
    cfg, inp, cache = _small_cache()
    rng = np.random.default_rng(4)
    for t in [2048, 3000, 6143, 8191]:
        q = O.normalise(rng.standard_normal((4, 64)))
        lr, info = O.select_flat(q, cache, t, 10 ** 9, 4, 128)
        nvis, sink_end, l0 = O.query_geometry(t, cache["n_blocks"], 4, 128)
        assert list(lr) == list(range(sink_end, l0))


def test_select_count_is_min_k_eligible():
    cfg, inp, cache = _small_cache()
    rng = np.random.default_rng(6)
    for t in [2048, 4100, 8191]:
        q = O.normalise(rng.standard_normal((4, 64)))
        lr, _ = O.select_flat(q, cache, t, 256, 4, 128)
        nvis, sink_end, l0 = O.query_geometry(t, cache["n_blocks"], 4, 128)
        assert len(lr) == min(256, max(0, l0 - sink_end))
        assert np.all(np.diff(lr) > 0)
        assert np.all((lr >= sink_end) & (lr < l0))


def test_tree_full_beam_equals_flat():
    cfg, inp, cache = _small_cache(tree=True, dtype="bf16")
    rng = np.random.default_rng(8)
    for t in [2048, 4500, 6200, 8191]:
        q = O.round_to(O.normalise(rng.standard_normal((4, 64))), "bf16")
        for k in [1, 37, 256, 5000]:
            lf, _ = O.select_flat(q, cache, t, k, 4, 128)
            lt, _ = O.select_tree(q, cache, t, k, 4, 128, beam=len(cache["sums"]))
            assert np.array_equal(lf, lt), (t, k)


def test_tree_hand_checkable_beam_one():
    # 4 leaves: root -> {n(1,0) = leaves 0,1 ; n(1,1) = leaves 2,3}
    sums = np.array([[1.0, 0, 0], [0.8, 0.6, 0], [0, 0, 1.0], [0, 0.6, 0.8]])
    sums = np.pad(sums, ((0, 0), (0, 61)))
    levels = O.build_tree(sums, "f64")
    members = [np.arange(8 * x, 8 * x + 8) for x in range(4)]
    cache = dict(n_blocks=1, members=members, sizes=np.full(4, 8), cent=O.normalise(sums), tree=levels)
    # LEAVES_PER_BLOCK = 64 leaves per block in general; only 4 exist here, all in block 0
    q = np.zeros((1, 64))
    q[0, 2] = 1.0        # prefers the (2,3) side, then leaf 2 (score 1.0) over leaf 3 (0.8)
    lr, info = O.select_tree(q, cache, t=4096, k=8, n_sinks=0, window=1, beam=1)
    assert list(info["ranked"]) == [2]
    assert list(lr) == list(range(64, 72))
    q[0, 2] = 0.0
    q[0, 1] = 1.0        # node(1,1) centroid ~(0,.6,1.8)/n vs node(1,0) ~(1.8,.6,0)/n: tie 0.3 vs 0.3 -> index 0
    lr, info = O.select_tree(q, cache, t=4096, k=8, n_sinks=0, window=1, beam=1)
    assert list(info["ranked"]) == [1]


def test_causal_tree_equals_the_tree_over_the_visible_blocks():
    """causal=True at position t is the plain tree search on the cache of the first nvis(t) blocks only
    (ch.2: blocks are clustered as the keys stream in, so a decode step at t sees exactly that tree):
    the truncated cache goes through build_tree, not through the partial-node sums."""
    from synth import get_config, layer_inputs
    cfg = get_config(1, T=2048 * 11 + 300)
    inp = layer_inputs(cfg, seed=41)
    W = inp["W"].double().numpy()
    Kg = inp["K"][0, 0].double().numpy()
    full = O.build_head_cache(Kg, W, "f32", tree=True, processes=8)
    rng = np.random.default_rng(12)
    changed = 0
    for nvis in (3, 5, 6, 7, 9, 11):
        trunc = O.build_head_cache(Kg[: nvis * 2048], W, "f32", tree=True, clusters=full["clusters"][:nvis])
        for t in (nvis * 2048 + 17, nvis * 2048 + 2000):
            q = O.round_to(O.normalise(rng.standard_normal((4, 64))), "f32")
            for beam in (1, 3, 8):
                a, _ = O.select_tree(q, full, t, 256, 4, 128, beam, causal=True)
                b, _ = O.select_tree(q, trunc, t, 256, 4, 128, beam)
                assert np.array_equal(a, b), (nvis, t, beam)
                c, _ = O.select_tree(q, full, t, 256, 4, 128, beam)
                changed += not np.array_equal(a, c)
    print(f"[causal tree] {changed} of 36 selections differ from the stored-centroid search")
    # the partial nodes do differ from the stored ones (the mode is not a no-op on this cache)
    m = 64 * 5
    lev = full["tree"][8]
    j = (m - 1) // lev["span"]
    part = O.round_to(O.normalise(full["sums"][j * lev["span"]: m].sum(axis=0)[None, :]), "f32")[0]
    assert not np.allclose(part, lev["cent"][j])


# ---------------------------------------------------------------- attention

def _sdpa(q, K, V, mask, scale):
    qt = torch.from_numpy(q).unsqueeze(0)
    Kt = torch.from_numpy(K).unsqueeze(0)
    Vt = torch.from_numpy(V).unsqueeze(0)
    m = torch.from_numpy(mask).unsqueeze(0)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m, scale=scale)[0].numpy()


def test_full_budget_equals_dense_causal_attention():
    cfg, inp, cache = _small_cache()
    K = inp["K"][0, 0].double().numpy()
    V = inp["V"][0, 0].double().numpy()
    Q = inp["Q"][0, :, :, :].double().numpy()
    W = inp["W"].double().numpy()
    scale = 1 / math.sqrt(cfg.d)
    for t in [0, 1, 2047, 2048, 5000, 8191]:
        qg = Q[t]
        qh = O.query_latent(qg, W, "f32")
        lr, _ = O.select_flat(qh, cache, t, 10 ** 9, cfg.n_sinks, cfg.window)
        ours = O.attend(qg, K, V, t, lr, cfg.n_sinks, cfg.window, cache["n_blocks"], scale)
        mask = np.zeros((qg.shape[0], len(K)), dtype=bool)
        mask[:, : t + 1] = True
        ref = _sdpa(qg, K, V, mask, scale)
        assert np.allclose(ours, ref, atol=1e-12), t


def test_zero_budget_is_sink_plus_local_attention():
    cfg, inp, cache = _small_cache()
    K = inp["K"][0, 0].double().numpy()
    V = inp["V"][0, 0].double().numpy()
    Q = inp["Q"][0].double().numpy()
    scale = 1 / math.sqrt(cfg.d)
    for t in [3, 2500, 8191]:
        nvis, sink_end, l0 = O.query_geometry(t, cache["n_blocks"], cfg.n_sinks, cfg.window)
        ours = O.attend(Q[t], K, V, t, np.zeros(0, np.int64), cfg.n_sinks, cfg.window, cache["n_blocks"], scale)
        mask = np.zeros((Q.shape[1], len(K)), dtype=bool)
        mask[:, :sink_end] = True
        mask[:, l0: t + 1] = True
        ref = _sdpa(Q[t], K, V, mask, scale)
        assert np.allclose(ours, ref, atol=1e-12)


def test_single_key_returns_its_value():
    K = np.random.default_rng(0).standard_normal((10, 8))
    V = np.random.default_rng(1).standard_normal((10, 8))
    out = O.attend(np.ones((3, 8)), K, V, 0, np.zeros(0, np.int64), 4, 16, 0, 0.3)
    assert np.allclose(out, V[0][None, :].repeat(3, 0))


def test_needle_is_retrieved():
    # decode at context 16384 with a planted needle; the needle's 4 tokens must be selected
    from synth import decode_inputs, get_config
    cfg = get_config(3, T=16384, B=2, H_kv=2, H_q=10, n_topics=64, window=256)
    inp = decode_inputs(cfg, seed=11)
    W = inp["W"].double().numpy()
    for b in range(cfg.B):
        p = inp["needle_pos"][b]
        for g in range(cfg.H_kv):
            K = inp["K"][b, g].double().numpy()
            cache = O.build_head_cache(K, W, "bf16", T=cfg.T)
            qh = O.query_latent(inp["Q"][b, 0, g * cfg.G:(g + 1) * cfg.G].double().numpy(), W, "bf16")
            lr, info = O.select_flat(qh, cache, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
            assert set(range(p, p + 4)) <= set(lr.tolist()), (b, g, p)


# ---------------------------------------------------------------- training-free projection (PCA)

def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_pca_closed_form_axes():
    """Keys whose covariance is exactly diagonal (orthogonal zero-mean Hadamard columns scaled by
    distinct sigmas): the principal directions are the axes of the largest sigmas, in that order."""
    H = _hadamard(16)[:, 1:9]                 # 16 x 8, zero-mean, orthogonal columns
    sig = np.array([0.3, 2.0, 0.7, 1.5, 0.1, 1.1, 0.5, 0.9])
    X = H * sig + 0.25                         # a constant shift must not matter
    W, lam = O.pca_projection(X, n_dir=3)
    axes = np.argsort(-sig)[:3]                # 1, 3, 5
    for j, ax in enumerate(axes):
        e = np.zeros(8)
        e[ax] = 1.0
        assert abs(abs(W[:, j] @ e) - 1.0) < 1e-12
    assert np.allclose(lam, np.sort(sig ** 2)[::-1], atol=1e-12)


def test_pca_rotation_equivariant_and_orthonormal():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((4000, 12)) * np.linspace(3.0, 0.2, 12)
    R, _ = np.linalg.qr(rng.standard_normal((12, 12)))
    W, _ = O.pca_projection(X, n_dir=5)
    W2, _ = O.pca_projection(X @ R, n_dir=5)
    assert np.allclose(W.T @ W, np.eye(5), atol=1e-12)
    assert np.allclose(W2 @ W2.T, R.T @ (W @ W.T) @ R, atol=1e-8)


def test_pca_captures_the_most_variance():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3000, 10)) @ rng.standard_normal((10, 10))
    W, lam = O.pca_projection(X, n_dir=4)
    C = np.cov(X.T, bias=True)
    best = np.trace(W.T @ C @ W)
    assert abs(best - lam[:4].sum()) < 1e-9 * lam[0]
    for _ in range(20):
        Qr, _ = np.linalg.qr(rng.standard_normal((10, 4)))
        assert np.trace(Qr.T @ C @ Qr) <= best + 1e-9


# ---------------------------------------------------------------- margins of the protocol

def test_boundary_margin_ignores_exact_ties():
    """Two leaves with the same centroid as the boundary leaf tie exactly (decided by id on both sides);
    the margin is the least nonzero gap, here to a leaf 3e-4 below."""
    cache = _hand_cache()
    cache["cent"][7] = cache["cent"][3]
    cache["cent"][9] = O.normalise(cache["cent"][3] - np.eye(64)[1] * 1e-3)   # slightly below in score
    q = cache["cent"][3][None, :].copy()
    # k = 32 tokens: leaf 3 (entries 24..31 = tokens 96..127) is the first and the boundary leaf
    lr, info = O.select_flat(q, cache, 4096, k=32, n_sinks=0, window=1, with_margin=True)
    assert info["boundary"] == 3 and list(lr) == list(range(96, 128))
    s = info["scores"]
    assert s[7] == s[3]
    others = np.delete(np.abs(s - s[3]), [3, 7])
    assert info["margin"] == pytest.approx(others.min()) and info["margin"] > 0


def test_cut_margin_around_exact_ties():
    # no tie at the cut: lowest kept minus highest dropped
    assert O.lsa_oracle._cut_margin([0.9, 0.5], [0.4, 0.1]) == pytest.approx(0.1)
    # a tie at the cut (0.5 kept and dropped, broken by index): the nearest distinct scores decide
    assert O.lsa_oracle._cut_margin([0.9, 0.5003, 0.5], [0.5, 0.45]) == pytest.approx(3e-4)
    assert O.lsa_oracle._cut_margin([0.9, 0.5], [0.5, 0.4999]) == pytest.approx(1e-4)
    # only tied values on both sides: nothing can reorder them
    assert O.lsa_oracle._cut_margin([0.5, 0.5], [0.5]) == math.inf
