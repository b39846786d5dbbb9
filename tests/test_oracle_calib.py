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


# ------------------------------------------------------------------------------------------------
# Head-block clustering of the SSD x channels (the 8 groups per head block reading): brute force
# over every labelling of each block's channels, independent of the sort and the DP.

def brute_force_block(absmax, G):
    """Least-cost assignment of the channels of one block to G non-empty groups (sum over groups
    of the squared deviations from the group mean), over all G^C labellings; the groups are then
    numbered by ascending magnitude. Returns (labels, cost)."""
    C = absmax.size
    v = absmax.astype(np.float64)
    best = None
    for lab in itertools.product(range(G), repeat=C):
        lab = np.asarray(lab)
        if len(set(lab.tolist())) != G:
            continue
        cost = sum(float(((v[lab == g] - v[lab == g].mean()) ** 2).sum()) for g in range(G))
        if best is None or cost < best[1] - 1e-12:
            best = (lab, cost)
    lab, cost = best
    order = np.argsort([v[lab == g].mean() for g in range(G)])
    rank = np.empty(G, int)
    rank[order] = np.arange(G)
    return rank[lab], cost


@pytest.mark.parametrize("nheads,headdim,ngroups,gpb,seed", [(4, 3, 2, 2, 0), (2, 4, 1, 3, 1),
                                                             (6, 2, 3, 2, 2), (3, 3, 1, 3, 3)])
def test_calib_ssd_x_matches_brute_force(nheads, headdim, ngroups, gpb, seed):
    import oracle.pipelines as op
    r = np.random.default_rng(seed)
    # calibration draw [T, nh, P] with a distinct spread per channel (no ties in the absmax)
    spread = np.exp(r.uniform(-2.0, 2.0, nheads * headdim))
    x_cal = (r.standard_normal((17, nheads, headdim)) *
             spread.reshape(nheads, headdim)).astype(np.float32)
    group_of, scales = op.calib_ssd_x(x_cal, nheads, headdim, ngroups, gpb)
    C = nheads * headdim
    per_block = C // ngroups
    absmax = np.abs(x_cal.reshape(-1, C)).max(axis=0)      # channel c = h * P + p
    assert len(set(absmax.tolist())) == C
    want_scales = np.zeros(ngroups * gpb, np.float32)
    for k in range(ngroups):
        blk = absmax[k * per_block:(k + 1) * per_block]
        lab, _ = brute_force_block(blk, gpb)
        assert np.array_equal(group_of[k * per_block:(k + 1) * per_block], lab + k * gpb), k
        for g in range(gpb):
            # scale = fl32(group absmax / 127), computed here from the exact quotient
            want_scales[k * gpb + g] = np.float32(np.float64(blk[lab == g].max()) / 127.0)
    assert np.array_equal(scales, want_scales)
