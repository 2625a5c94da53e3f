"""Pins of the oracle's source-range split of the heavy rows (plan option
xcd_split): a hand-worked example, and the properties its definition fixes
on random graphs (each heavy row covered exactly once in order, every group
within one source range and at most C entries, near-equal groups inside a
range's part, and the launch order's slot i*8 + r holding range r's i-th
group)."""
import numpy as np
import pytest

import oracle


def test_hand_worked_example():
    # N = 16, so R = 2 ids per range. Row 3 (entries 10..16) lists sources
    # 0 1 | 3 | 4 5 | 9 | 15 in ranges 0, 1, 2, 4, 7; row 7 (entries 17..21)
    # lists source 2 five times (range 1). C = 2: the five entries of row 7
    # in range 1 make ceil(5/2) = 3 groups [17,18) [18,20) [20,22)
    # (17 + 5*j//3 for j = 0..3 gives 17, 18, 20, 22).
    rows = {0: [0, 1, 2, 3, 4], 1: [1, 2, 3], 2: [5, 6], 3: [0, 1, 3, 4, 5, 9, 15], 7: [2, 2, 2, 2, 2]}
    deg = np.zeros(16, np.int64)
    for r, v in rows.items():
        deg[r] = len(v)
    ip = np.concatenate([[0], np.cumsum(deg)])
    ix = np.concatenate([rows[r] for r in sorted(rows)]).astype(np.int32)
    assert ip[3] == 10 and ip[7] == 17 and ip[16] == 22
    x = oracle.xsplit(ip, ix, np.array([3, 7]), 16, chunk=2)
    want_groups = [(3, 10, 12), (3, 12, 13), (3, 13, 15), (3, 15, 16), (3, 16, 17),
                   (7, 17, 18), (7, 18, 20), (7, 20, 22)]
    assert x["groups"].tolist() == [list(g) for g in want_groups]
    assert x["partial_ofs"].tolist() == [0, 5, 8]
    # ranges of the groups: 0 1 2 4 7 | 1 1 1; range 1 has the most (4), so 32 slots
    want_order = [0, 1, 2, -1, 3, -1, -1, 4] + [-1, 5] + [-1] * 6 + [-1, 6] + [-1] * 6 + [-1, 7] + [-1] * 6
    assert x["order"].tolist() == want_order


def _sorted_random_graph(rng, n, hubs):
    deg = rng.poisson(6, n)
    deg[rng.choice(n, hubs, replace=False)] = rng.integers(300, max(301, 3 * n), hubs)
    rows = [np.sort(rng.integers(0, n, d)) for d in deg]
    ip = np.concatenate([[0], np.cumsum(deg)])
    return ip, np.concatenate(rows).astype(np.int32)


@pytest.mark.parametrize("seed,n,chunk,waves", [(1, 1000, 64, 4), (2, 777, 7, 2), (3, 4096, 512, 1), (4, 9, 1, 1)])
def test_properties(seed, n, chunk, waves):
    rng = np.random.default_rng(seed)
    ip, ix = _sorted_random_graph(rng, n, hubs=min(5, n))
    heavy = oracle.bucketing(ip, 100, chunk, waves)["heavy"]
    x = oracle.xsplit(ip, ix, heavy, n, chunk)
    g, pofs, order = x["groups"].astype(np.int64), x["partial_ofs"], x["order"]
    R, span = -(-n // 8), chunk
    assert pofs[0] == 0 and pofs[-1] == len(g) and np.all(np.diff(pofs) >= 1)
    rng_of = np.empty(len(g), np.int64)
    for k, node in enumerate(heavy):
        mine = g[pofs[k]:pofs[k + 1]]
        assert np.all(mine[:, 0] == node)
        # the node's entries, covered once and in order
        assert mine[0, 1] == ip[node] and mine[-1, 2] == ip[node + 1] and np.all(mine[1:, 1] == mine[:-1, 2])
        sizes = mine[:, 2] - mine[:, 1]
        assert np.all(sizes >= 1) and np.all(sizes <= span)
        for i, (_, a, b) in enumerate(mine):
            r = np.unique(ix[a:b] // R)
            assert r.size == 1                     # one source range per group
            rng_of[pofs[k] + i] = r[0]
        # inside one range's part the groups differ in size by at most one
        for r in np.unique(rng_of[pofs[k]:pofs[k + 1]]):
            s = sizes[rng_of[pofs[k]:pofs[k + 1]] == r]
            assert s.max() - s.min() <= 1
    # launch order: slot 8i + r holds the i-th group of range r, then -1
    counts = np.bincount(rng_of, minlength=8)
    assert order.size == 8 * counts.max()
    for r in range(8):
        col = order[r::8]
        assert np.array_equal(col[:counts[r]], np.nonzero(rng_of == r)[0]) and np.all(col[counts[r]:] == -1)
