"""Pin of the oracle's channel clustering (Quamba2 step 2) against brute force over every
contiguous partition of the sorted channels. CPU only."""
import itertools

import numpy as np
import pytest

import oracle


def partition_cost(vals, bounds):
    cost = 0.0
    for a, b in zip(bounds[:-1], bounds[1:]):
        seg = np.asarray(vals[a:b], dtype=np.float64)
        cost += float(((seg - seg.mean()) ** 2).sum())
    return cost


def brute_force(vals, G):
    C = len(vals)
    best = None
    for cuts in itertools.combinations(range(1, C), G - 1):
        bounds = (0, *cuts, C)
        c = partition_cost(vals, bounds)
        if best is None or c < best[0] - 1e-12 * max(1.0, abs(best[0])):
            best = (c, bounds)
    return best


@pytest.mark.parametrize("C,G,seed", [(1, 1, 0), (5, 1, 1), (5, 5, 2), (8, 3, 3), (10, 4, 4),
                                      (12, 4, 5), (12, 2, 6), (11, 3, 7)])
def test_cluster_matches_brute_force(C, G, seed):
    r = np.random.default_rng(seed)
    absmax = (np.exp(r.standard_normal(C) * 1.5)).astype(np.float32)
    perm, group_of = oracle.cluster_channels(absmax, G)
    assert np.array_equal(perm, np.argsort(absmax, kind="stable"))
    srt = absmax[perm].astype(np.float64)
    # groups are contiguous, ascending, non-empty, G of them
    assert group_of[0] == 0 and group_of[-1] == G - 1
    assert np.all(np.diff(group_of.astype(int)) >= 0) and np.all(np.diff(group_of.astype(int)) <= 1)
    bounds = (0, *[int(i) for i in np.nonzero(np.diff(group_of.astype(int)))[0] + 1], C)
    best_cost, best_bounds = brute_force(srt, G)
    assert partition_cost(srt, bounds) == pytest.approx(best_cost, rel=1e-9, abs=1e-12)
    assert bounds == best_bounds


def test_cluster_separates_obvious_groups():
    absmax = np.array([100.0, 1.0, 1.1, 50.0, 0.9, 51.0, 99.0], dtype=np.float32)
    perm, group_of = oracle.cluster_channels(absmax, 3)
    assert absmax[perm].tolist() == sorted(absmax.tolist())
    assert group_of.tolist() == [0, 0, 0, 1, 1, 2, 2]


def test_cluster_ties_keep_stable_order():
    absmax = np.array([2.0, 1.0, 2.0, 1.0], dtype=np.float32)
    perm, group_of = oracle.cluster_channels(absmax, 2)
    assert perm.tolist() == [1, 3, 0, 2]
    assert group_of.tolist() == [0, 0, 1, 1]
