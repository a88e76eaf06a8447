"""Plain float64 oracle of the Latent Sparse Attention (LSA) layer.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the CPU-baseline
leg of bench.py, never by the library.  It shares no code with the HIP path.

Sources (the pages' titles and sections):
  * zhichai.net, "卡片柜 — 当注意力学会先查目录再翻书":
      ch.2 (semantic clustering): 64-d latent projection, L2 normalisation,
        pooling 4 consecutive keys, Ward clustering inside 512-entry blocks to
        buckets of mean 8 / max 16 members, normalised-mean centroids kept in a
        bucket cache, clustering done once per block and never revisited;
      ch.3 (query path): score every centroid, take the top-p buckets and
        expand them until k long-range keys, plus sinks and a local window;
      ch.4 (tree): a complete binary tree whose nodes merge two siblings and
        whose centroid is the mean of all keys below, searched level by level;
      ch.5 (D-/N-LSA): separate key/query projections; a bucket's score is the
        max over heads.
  * diosapp.com.cn LSA tutorial, section 二, pseudocode: the query is projected
    by the same map and the output is softmax(q K[keys]^T / sqrt(d)) V[keys].
  * zhichai.net explainer, ch.5 (the training-free D-LSA variant): the
    projection is taken as the leading 64 principal directions of the keys.

Readings taken where the pages are silent:
  a block is 512 pooled entries = 2048 tokens; pooling is the plain mean of
  the 4 unit latents (no renormalisation); the Ward stop is ceil(n / 8)
  clusters, a merge is allowed only if the union has <= 16 entries, ties go to
  the lexicographically lowest (id_A, id_B) with a cluster's id its smallest
  member; leaves of a block are numbered by id, globally 64 * block + rank;
  stored centroids and query latents are rounded (round-to-nearest-even) to
  the storage dtype before scoring; only blocks strictly before the query's
  block are selectable and the query's own unbucketed block is attended
  densely (the local window is widened to its start); leaves are ranked by
  (score desc, id asc) and taken whole, the boundary leaf contributing its
  lowest-index eligible tokens; tree nodes pair (2j, 2j+1) level by level, an
  odd last node is carried up alone, and beam search keeps the best `beam`
  visible children by (score desc, index asc) at each level.
"""

from __future__ import annotations

import math
import multiprocessing as mp
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "POOL", "BLOCK_ENTRIES", "BLOCK_TOKENS", "MEAN_BUCKET", "MAX_BUCKET", "LEAVES_PER_BLOCK",
    "round_to", "normalise", "key_latents", "pooled_entries", "ward_block", "ward_blocks",
    "build_head_cache", "build_tree", "query_latent", "query_geometry", "leaf_tokens",
    "eligible_tokens", "select_flat", "select_tree", "attend", "attend_set", "pca_projection",
]

POOL = 4
BLOCK_ENTRIES = 512
BLOCK_TOKENS = POOL * BLOCK_ENTRIES          # 2048 tokens per cluster block
MEAN_BUCKET = 8
MAX_BUCKET = 16
LEAVES_PER_BLOCK = BLOCK_ENTRIES // MEAN_BUCKET   # 64


# --------------------------------------------------------------------------
# rounding and normalisation
# --------------------------------------------------------------------------

def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to the storage precision, to nearest even.

    'f32' uses NumPy's float32 cast (IEEE round-to-nearest-even); 'bf16' keeps
    8 significant bits: x = m 2^e with 1/2 <= |m| < 1, m is scaled by 2^8,
    rounded half-to-even and scaled back.  'f64' returns x unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(x)
        return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    raise ValueError(dtype)


def normalise(x: np.ndarray) -> np.ndarray:
    """Rows divided by their L2 norm; a zero row stays zero."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    out = np.zeros_like(x)
    np.divide(x, n, out=out, where=n > 0)
    return out


# --------------------------------------------------------------------------
# key side: latent, pooling, Ward, centroids, tree
# --------------------------------------------------------------------------

def key_latents(Kg: np.ndarray, W: np.ndarray) -> np.ndarray:
    """u_t = z_t / ||z_t||, z_t = K[t] W  (ch.2: 64-d projection then L2 norm)."""
    return normalise(np.asarray(Kg, np.float64) @ np.asarray(W, np.float64))


def pooled_entries(u: np.ndarray) -> np.ndarray:
    """e_i = mean of u_{4i}..u_{4i+3}; a trailing partial group is dropped (ch.2)."""
    u = np.asarray(u, np.float64)
    n = len(u) // POOL
    if n == 0:
        return np.zeros((0, u.shape[1] if u.ndim == 2 else 0))
    return u[: n * POOL].reshape(n, POOL, -1).mean(axis=1)


def _ward_pair_cost(size_a, mu_a, sizes, mus):
    return size_a * sizes / (size_a + sizes) * ((mus - mu_a) ** 2).sum(axis=1)


def ward_block(E: np.ndarray, cap: int = MAX_BUCKET, mean_bucket: int = MEAN_BUCKET,
               target: Optional[int] = None, margins: bool = False) -> Dict:
    """Greedy capped Ward clustering of one block of pooled entries (ch.2).

    Start from singletons; while there are more than `target` (default
    ceil(n / mean_bucket)) clusters, merge the allowed pair with the least
    increase of the within-cluster sum of squares,
        delta(A, B) = |A||B| / (|A| + |B|) * ||mean_A - mean_B||^2,
    a pair being allowed when |A| + |B| <= cap.  Ties go to the lowest
    (id_A, id_B), id = smallest member.  The delta of every live pair is held
    in an n x n upper-triangular table; after a merge only the pairs of the
    merged cluster are recomputed (every other pair is unchanged), from the
    merged cluster's mean taken over its members.

    Returns dict(clusters=[sorted member lists, by id], heights=[delta per
    merge]) and, with margins=True, merges=[(a, b, delta, conflict_gap,
    global_gap)] where conflict_gap is the least delta of another allowed pair
    sharing a or b minus delta, global_gap the second-least delta overall minus
    delta; and stop_gap = least remaining allowed delta minus the last delta.
    """
    E = np.asarray(E, np.float64)
    n = len(E)
    if target is None:
        target = -(-n // mean_bucket)
    target = max(1, min(n, target))
    members: List[List[int]] = [[i] for i in range(n)]
    size = np.ones(n)
    mu = E.copy()
    active = np.ones(n, dtype=bool)
    D = np.full((n, n), np.inf)
    if cap >= 2:
        for i in range(n - 1):
            D[i, i + 1:] = 0.5 * ((E[i + 1:] - E[i]) ** 2).sum(axis=1)
    heights: List[float] = []
    merges = []
    n_active = n
    while n_active > target:
        flat = int(np.argmin(D))
        a, b = divmod(flat, n)
        dab = float(D[a, b])
        if not np.isfinite(dab):
            raise RuntimeError("no allowed pair left before reaching the target")
        if margins:
            D[a, b] = np.inf
            conflict = min(D[a].min(), D[:, a].min(), D[b].min(), D[:, b].min())
            glob = D.min()
            D[a, b] = dab
            merges.append((a, b, dab, conflict - dab, glob - dab))
        heights.append(dab)
        members[a] = sorted(members[a] + members[b])
        members[b] = []
        size[a] += size[b]
        size[b] = 0
        active[b] = False
        mu[a] = E[members[a]].mean(axis=0)
        D[b, :] = np.inf
        D[:, b] = np.inf
        others = np.flatnonzero(active)
        others = others[others != a]
        if len(others):
            dl = _ward_pair_cost(size[a], mu[a], size[others], mu[others])
            dl = np.where(size[a] + size[others] <= cap, dl, np.inf)
            lo = others < a
            D[others[lo], a] = dl[lo]
            D[a, others[~lo]] = dl[~lo]
        n_active -= 1
    out = dict(clusters=[members[i] for i in range(n) if active[i]], heights=heights)
    if margins:
        out["merges"] = merges
        out["stop_gap"] = (float(D.min()) - heights[-1]) if heights else math.inf
    return out


def _ward_job(args):
    E, cap, mean_bucket = args
    return ward_block(E, cap=cap, mean_bucket=mean_bucket)["clusters"]


def ward_blocks(E_blocks: Sequence[np.ndarray], processes: int = 1) -> List[List[List[int]]]:
    """ward_block over independent blocks, optionally in a process pool."""
    jobs = [(E, MAX_BUCKET, MEAN_BUCKET) for E in E_blocks]
    if processes <= 1 or len(jobs) <= 1:
        return [_ward_job(j) for j in jobs]
    ctx = mp.get_context("fork")
    with ctx.Pool(processes) as pool:
        return pool.map(_ward_job, jobs, chunksize=max(1, len(jobs) // (4 * processes)))


def build_head_cache(Kg: np.ndarray, W: np.ndarray, dtype: str, T: Optional[int] = None,
                     tree: bool = False, processes: int = 1, clusters=None) -> Dict:
    """Bucket cache of one (sequence, KV head): every full 2048-token block.

    Leaves of block b are its Ward clusters ordered by id; global leaf id
    64 b + rank.  sums[x] = sum of the member entries, cent[x] =
    round(sums[x] / ||sums[x]||) in the storage dtype (ch.2: the normalised
    mean of the bucket's keys is its card).  `clusters` may pass in the
    per-block clusters already computed by this module.
    """
    Kg = np.asarray(Kg, np.float64)
    T = len(Kg) if T is None else T
    nb = T // BLOCK_TOKENS
    u = key_latents(Kg[: nb * BLOCK_TOKENS], W)
    e = pooled_entries(u)
    if clusters is None:
        clusters = ward_blocks([e[b * BLOCK_ENTRIES:(b + 1) * BLOCK_ENTRIES] for b in range(nb)], processes)
    members, block_of = [], []
    for b, cl in enumerate(clusters):
        for c in cl:
            members.append(np.asarray(c, dtype=np.int64) + b * BLOCK_ENTRIES)
            block_of.append(b)
    NL = len(members)
    sums = np.zeros((NL, e.shape[1] if len(e) else 64))
    for x, m in enumerate(members):
        sums[x] = e[m].sum(axis=0)
    cache = dict(n_blocks=nb, dtype=dtype, members=members, sizes=np.array([len(m) for m in members], dtype=np.int64),
                 block=np.array(block_of, dtype=np.int64), sums=sums, cent=round_to(normalise(sums), dtype),
                 entries=e, clusters=clusters)
    if tree:
        cache["tree"] = build_tree(sums, dtype)
    return cache


def build_tree(sums: np.ndarray, dtype: str) -> List[Dict]:
    """Complete binary tree over the leaves (ch.4).

    Level 0 holds the leaves in id order; node (l, j) covers leaves
    [j 2^l, min((j+1) 2^l, NL)), i.e. children (l-1, 2j) and (l-1, 2j+1) when
    they exist.  Its sum is the sum of the covered leaves' sums and its
    centroid round(sum / ||sum||).  Levels continue until one node is left.
    """
    NL = len(sums)
    levels = []
    lev = 0
    while True:
        span = 1 << lev
        starts = np.arange(0, NL, span)
        s = np.add.reduceat(sums, starts, axis=0) if NL else np.zeros((0, sums.shape[1]))
        levels.append(dict(sums=s, cent=round_to(normalise(s), dtype), first_leaf=starts, span=span))
        if len(starts) <= 1:
            break
        lev += 1
    return levels


# --------------------------------------------------------------------------
# query side
# --------------------------------------------------------------------------

def query_latent(Qg: np.ndarray, W: np.ndarray, dtype: str) -> np.ndarray:
    """q_hat = round(normalise(q W)) for each query head of the group (ch.5, 二)."""
    return round_to(normalise(np.asarray(Qg, np.float64) @ np.asarray(W, np.float64)), dtype)


def query_geometry(t: int, n_blocks: int, n_sinks: int, window: int):
    """(nvis, sink_end, l0) for a query at position t.

    nvis: blocks selectable (those strictly before the query's block, and
    built); sinks = [0, sink_end); local = [l0, t], the last `window` tokens
    widened back to the first unselectable token.
    """
    nvis = min(t // BLOCK_TOKENS, n_blocks)
    sink_end = min(n_sinks, t + 1)
    l0 = max(0, min(t - window + 1, BLOCK_TOKENS * nvis))
    return nvis, sink_end, l0


def leaf_tokens(members: np.ndarray) -> np.ndarray:
    """Tokens of a leaf: {4i, 4i+1, 4i+2, 4i+3 : i a member entry}, ascending."""
    m = np.sort(np.asarray(members, np.int64))
    return (m[:, None] * POOL + np.arange(POOL)[None, :]).reshape(-1)


def eligible_tokens(members, t: int, sink_end: int, l0: int) -> np.ndarray:
    """Leaf tokens minus the sinks [0, sink_end) and the local window [l0, t]."""
    tok = leaf_tokens(members)
    in_sink = tok < sink_end
    in_local = (tok >= l0) & (tok <= t)
    return tok[~(in_sink | in_local)]


def _walk(ranked: Sequence[int], scores: np.ndarray, members, t, sink_end, l0, k):
    """Take ranked leaves whole until k eligible tokens; the boundary leaf gives
    its lowest-index eligible tokens.  Returns (sorted LR, boundary leaf or None)."""
    out: List[np.ndarray] = []
    have = 0
    boundary = None
    for x in ranked:
        if have >= k:
            break
        tok = eligible_tokens(members[x], t, sink_end, l0)
        if len(tok) == 0:
            continue
        take = tok[: k - have]
        out.append(take)
        have += len(take)
        if have >= k:
            boundary = x
    lr = np.sort(np.concatenate(out)) if out else np.zeros(0, dtype=np.int64)
    return lr.astype(np.int64), boundary


def _boundary_margin(boundary, scores, weights_positive):
    """Least nonzero |score(x) - score(boundary)| over the other leaves that hold
    eligible tokens.  An exact tie (gap 0) is not a margin: it is decided by the
    lowest-id rule, and both sides compute equal scores for equal centroids."""
    if boundary is None:
        return math.inf
    others = np.flatnonzero(weights_positive)
    others = others[others != boundary]
    if len(others) == 0:
        return math.inf
    gaps = np.abs(scores[others] - scores[boundary])
    gaps = gaps[gaps > 0]
    return float(gaps.min()) if len(gaps) else math.inf


def _cut_margin(kept_scores, dropped_scores):
    """Least nonzero gap between a kept and a dropped score at a beam cut.
    Without a tie at the cut it is the lowest kept minus the highest dropped
    score; with an exact tie there (broken by index) the nearest distinct
    scores on either side of the tied value decide."""
    kept = np.asarray(kept_scores, np.float64)
    dropped = np.asarray(dropped_scores, np.float64)
    if len(kept) == 0 or len(dropped) == 0:
        return math.inf
    kmin, dmax = float(kept.min()), float(dropped.max())
    if kmin > dmax:
        return kmin - dmax
    above, below = kept[kept > kmin], dropped[dropped < kmin]
    gaps = ([float(above.min()) - kmin] if len(above) else []) + ([kmin - float(below.max())] if len(below) else [])
    return min(gaps) if gaps else math.inf


def _weights_positive(cache, NLv, t, sink_end, l0):
    return np.array([len(eligible_tokens(cache["members"][x], t, sink_end, l0)) > 0 for x in range(NLv)],
                    dtype=bool)


def select_flat(qhat: np.ndarray, cache: Dict, t: int, k: int, n_sinks: int, window: int,
                with_margin: bool = False):
    """Flat search (ch.3): score every visible leaf, rank, expand to k tokens.

    score(x) = max over the group's query heads of <q_hat_h, c_x> (ch.5 takes
    the max over heads).  Returns (LR int64 ascending, info dict with
    'boundary', 'scores', 'ranked' and, if asked, 'margin' = the least
    nonzero |score(x) - score(boundary)| over other visible leaves with eligible
    tokens; exact ties are decided by the lowest-id rule).
    """
    nvis, sink_end, l0 = query_geometry(t, cache["n_blocks"], n_sinks, window)
    NLv = LEAVES_PER_BLOCK * nvis
    info = dict(nvis=nvis, l0=l0, sink_end=sink_end, boundary=None, margin=math.inf)
    if NLv == 0 or k <= 0:
        return np.zeros(0, dtype=np.int64), info
    scores = (cache["cent"][:NLv] @ np.asarray(qhat, np.float64).T).max(axis=1)
    ids = np.arange(NLv)
    ranked = np.lexsort((ids, -scores))
    lr, boundary = _walk(ranked, scores, cache["members"], t, sink_end, l0, k)
    info.update(boundary=boundary, scores=scores, ranked=ranked)
    if with_margin:
        info["margin"] = _boundary_margin(boundary, scores, _weights_positive(cache, NLv, t, sink_end, l0))
    return lr, info


def select_tree(qhat: np.ndarray, cache: Dict, t: int, k: int, n_sinks: int, window: int, beam: int,
                with_margin: bool = False, causal: bool = False):
    """Tree search (ch.4): beam descent from the root, then expansion.

    A node is visible when its first leaf is visible; it is scored with its
    stored centroid, or, with causal=True, a node whose leaves are only
    partly visible is scored with the centroid of its visible leaves
    (round(normalise(sum of their sums))): the node as the tree over the
    blocks seen so far has it (ch.2: blocks are clustered as keys stream in).
    At each level the candidates are the visible children of the beam and the
    best `beam` by (score desc, index asc) are kept; the kept leaves are then
    expanded exactly as in the flat search.  info['cuts'] lists, per level
    with more candidates than the beam, the least nonzero gap between a kept
    and a dropped score (exact ties are decided by the index rule).
    """
    levels = cache["tree"]
    nvis, sink_end, l0 = query_geometry(t, cache["n_blocks"], n_sinks, window)
    NLv = LEAVES_PER_BLOCK * nvis
    info = dict(nvis=nvis, l0=l0, sink_end=sink_end, boundary=None, margin=math.inf, cuts=[])
    if NLv == 0 or k <= 0:
        return np.zeros(0, dtype=np.int64), info
    q = np.asarray(qhat, np.float64)
    top = len(levels) - 1
    frontier = np.array([0], dtype=np.int64)
    fscore = (levels[top]["cent"][frontier] @ q.T).max(axis=1)
    for lev in range(top - 1, -1, -1):
        n_lev = len(levels[lev]["first_leaf"])
        span = levels[lev]["span"]
        ch = np.concatenate([2 * frontier, 2 * frontier + 1])
        ch = np.unique(ch[(ch < n_lev) & (ch * span < NLv)])
        cent = levels[lev]["cent"][ch]
        if causal:
            for r, j in enumerate(ch):
                if (j + 1) * span > NLv:   # straddles the visible leaves
                    part = np.add.reduceat(cache["sums"][j * span: NLv], [0], axis=0)[0]
                    cent[r] = round_to(normalise(part[None, :]), cache["dtype"])[0]
        sc = (cent @ q.T).max(axis=1)
        order = np.lexsort((ch, -sc))
        if len(order) > beam:
            info["cuts"].append(_cut_margin(sc[order[:beam]], sc[order[beam:]]))
        keep = order[:beam]
        frontier, fscore = ch[keep], sc[keep]
    # frontier is ranked by (score desc, id asc) already
    leaf_scores = np.full(NLv, -np.inf)
    leaf_scores[frontier] = fscore
    lr, boundary = _walk(frontier, leaf_scores, cache["members"], t, sink_end, l0, k)
    info.update(boundary=boundary, ranked=frontier, frontier_scores=fscore)
    if with_margin:
        pos = np.zeros(NLv, dtype=bool)
        pos[frontier] = _weights_positive(cache, NLv, t, sink_end, l0)[frontier]
        m = _boundary_margin(boundary, leaf_scores, pos)
        info["margin"] = min([m] + [abs(c) for c in info["cuts"]])
    return lr, info


def attend_set(q: np.ndarray, Kg: np.ndarray, Vg: np.ndarray, S: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K[S]^T * scale) V[S] for each row of q, max subtracted (二)."""
    q = np.asarray(q, np.float64)
    if len(S) == 0:
        return np.zeros((q.shape[0], Vg.shape[1]))
    Ks = np.asarray(Kg[S], np.float64)
    Vs = np.asarray(Vg[S], np.float64)
    logits = (q @ Ks.T) * scale
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    return (p @ Vs) / p.sum(axis=1, keepdims=True)


def attend(q: np.ndarray, Kg: np.ndarray, Vg: np.ndarray, t: int, lr: np.ndarray, n_sinks: int,
           window: int, n_blocks: int, scale: float) -> np.ndarray:
    """Exact attention of the group's heads over S = sinks U local U LR (ch.3)."""
    nvis, sink_end, l0 = query_geometry(t, n_blocks, n_sinks, window)
    S = np.union1d(np.union1d(np.arange(sink_end), np.arange(l0, t + 1)), np.asarray(lr, np.int64))
    return attend_set(q, Kg, Vg, S.astype(np.int64), scale)


# --------------------------------------------------------------------------
# training-free projection (ch.5): principal directions of the keys
# --------------------------------------------------------------------------

def pca_projection(keys: np.ndarray, n_dir: int = 64):
    """Leading n_dir principal directions of a set of key rows (ch.5).

    keys: [N, d] (every key of every head and sequence of the layer).  The
    covariance is C = (1/N) sum (k - mean)(k - mean)^T in float64; its
    eigenvectors sorted by eigenvalue descending give W = [v_1 .. v_n_dir]
    ([d, n_dir], orthonormal columns).  Returns (W, all eigenvalues
    descending).  Only the spanned subspace is defined (signs, and rotations
    inside repeated eigenvalues, are arbitrary); the LSA path depends on W
    only through that subspace, since every latent is normalised.
    """
    X = np.asarray(keys, np.float64)
    mu = X.mean(axis=0)
    C = (X - mu).T @ (X - mu) / X.shape[0]
    lam, vec = np.linalg.eigh(C)
    order = np.argsort(-lam, kind="stable")
    return vec[:, order[:n_dir]], lam[order]

