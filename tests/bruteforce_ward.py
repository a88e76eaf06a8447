"""Brute-force capped Ward clustering, written independently of the oracle.

Every candidate pair's cost is recomputed from the point sets as
ESS(A u B) - ESS(A) - ESS(B) (no cached means, no update formula), where
ESS(S) = sum over S of ||x - mean(S)||^2 (Ward 1963, the objective named in
the zhichai.net explainer, ch.2: merge the pair whose union raises the total
variance least).  Used only to pin the oracle on small inputs.
"""

import numpy as np


def ess(points):
    points = np.asarray(points, dtype=np.float64)
    return float(((points - points.mean(axis=0)) ** 2).sum())


def brute_ward(E, cap, target):
    E = np.asarray(E, dtype=np.float64)
    clusters = [[i] for i in range(len(E))]
    while len(clusters) > target:
        best = None
        for ia in range(len(clusters)):
            for ib in range(ia + 1, len(clusters)):
                A, B = clusters[ia], clusters[ib]
                if len(A) + len(B) > cap:
                    continue
                cost = ess(E[A + B]) - ess(E[A]) - ess(E[B])
                key = (cost, min(A), min(B))
                if best is None or key < best[0]:
                    best = (key, ia, ib)
        if best is None:
            raise RuntimeError("no allowed pair")
        _, ia, ib = best
        merged = sorted(clusters[ia] + clusters[ib])
        clusters = [c for j, c in enumerate(clusters) if j not in (ia, ib)] + [merged]
        clusters.sort(key=min)
    return clusters
