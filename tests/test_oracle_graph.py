"""Pins for the oracle's integer structure (CSR, bucketing, CSC, tile census).

Each is checked against a brute-force Python construction written
independently from the definition, plus invariants that any correct result
satisfies."""
import numpy as np
import pytest

import oracle
from _helpers import random_graph


def _brute_csr(src, dst, n, self_loops):
    rows = [set() for _ in range(n)]
    for s, d in zip(src.tolist(), dst.tolist()):
        rows[d].add(s)
    if self_loops:
        for i in range(n):
            rows[i].add(i)
    indptr = [0]
    indices = []
    for i in range(n):
        r = sorted(rows[i])
        indices += r
        indptr.append(len(indices))
    return np.array(indptr, np.int32), np.array(indices, np.int32)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("self_loops", [True, False])
def test_csr_matches_brute_force(seed, self_loops):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    m = int(rng.integers(0, 200))
    src = rng.integers(0, n, m).astype(np.int32)
    dst = rng.integers(0, n, m).astype(np.int32)     # duplicates and self-pairs included
    ip, ix = oracle.csr_build(src, dst, n, add_self_loops=self_loops)
    bp, bx = _brute_csr(src, dst, n, self_loops)
    assert np.array_equal(ip, bp) and np.array_equal(ix, bx)
    # invariants
    assert ip[0] == 0 and ip[-1] == ix.size and np.all(np.diff(ip) >= 0)
    for i in range(n):
        r = ix[ip[i]:ip[i + 1]]
        assert np.all(np.diff(r) > 0)                  # strictly ascending, no duplicates
        if self_loops:
            assert np.count_nonzero(r == i) == 1


def test_csr_empty_and_isolated():
    ip, ix = oracle.csr_build(np.zeros(0, np.int32), np.zeros(0, np.int32), 5, add_self_loops=False)
    assert np.array_equal(ip, np.zeros(6, np.int32)) and ix.size == 0
    ip, ix = oracle.csr_build(np.zeros(0, np.int32), np.zeros(0, np.int32), 5, add_self_loops=True)
    assert np.array_equal(ip, np.arange(6)) and np.array_equal(ix, np.arange(5))


def test_csr_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.csr_build(np.array([0, 5]), np.array([1, 1]), 5)


def _brute_bucketing(indptr, T, C, W):
    light, heavy, groups, ofs = [], [], [], [0]
    for i in range(len(indptr) - 1):
        deg = indptr[i + 1] - indptr[i]
        if deg <= T:
            light.append(i)
            continue
        heavy.append(i)
        e = indptr[i]
        while e < indptr[i + 1]:
            groups.append((i, e, min(e + C * W, indptr[i + 1])))
            e += C * W
        ofs.append(len(groups))
    return light, heavy, groups, ofs


@pytest.mark.parametrize("T,C,W", [(0, 1, 1), (3, 2, 2), (5, 4, 1), (10 ** 9, 8, 4), (2, 3, 4), (1, 1, 8)])
def test_bucketing_matches_brute_force(T, C, W):
    rng = np.random.default_rng(T + C + W)
    n = 60
    deg = rng.integers(0, 30, n)
    deg[rng.integers(0, n, 5)] = 0
    indptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    b = oracle.bucketing(indptr, T, C, W)
    light, heavy, groups, ofs = _brute_bucketing(indptr.tolist(), T, C, W)
    assert b["light"].tolist() == light
    assert b["heavy"].tolist() == heavy
    assert [tuple(g) for g in b["groups"].tolist()] == groups
    assert b["partial_ofs"].tolist() == ofs
    # invariants: a partition of the nodes; groups tile each heavy row exactly
    allv = np.sort(np.concatenate([b["light"], b["heavy"]]))
    assert np.array_equal(allv, np.arange(n))
    for k, i in enumerate(b["heavy"]):
        g = b["groups"][b["partial_ofs"][k]:b["partial_ofs"][k + 1]]
        assert g[0, 1] == indptr[i] and g[-1, 2] == indptr[i + 1]
        assert np.all(g[1:, 1] == g[:-1, 2]) and np.all((g[:, 2] - g[:, 1]) <= C * W)
        assert np.all(g[:, 0] == i)


def test_degree_equal_threshold_is_light():
    indptr = np.array([0, 4, 9], np.int32)
    b = oracle.bucketing(indptr, 4, 2, 1)
    assert b["light"].tolist() == [0] and b["heavy"].tolist() == [1]


@pytest.mark.parametrize("seed", range(5))
def test_csc_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 50))
    src, dst, _ = random_graph(rng, n, p=0.2)
    ip, ix = oracle.csr_build(src, dst, n)
    cip, cix = oracle.csc(ip, ix, n)
    cols = [[] for _ in range(n)]
    for i in range(n):
        for j in ix[ip[i]:ip[i + 1]]:
            cols[j].append(i)
    assert cix.tolist() == sum((sorted(c) for c in cols), [])
    assert cip.tolist() == np.concatenate([[0], np.cumsum([len(c) for c in cols])]).tolist()
    # transposing twice gives the CSR back
    ip2, ix2 = oracle.csc(cip, cix, n)
    assert np.array_equal(ip2, ip) and np.array_equal(ix2, ix)


def test_csc_multigraph_keeps_multiplicity():
    indptr = np.array([0, 3, 4], np.int32)
    indices = np.array([1, 1, 0, 1], np.int32)
    cip, cix = oracle.csc(indptr, indices, 2)
    assert cip.tolist() == [0, 1, 4] and cix.tolist() == [0, 0, 0, 1]


def _brute_tiles(indptr, indices, n, min_nnz):
    cnt = {}
    for i in range(n):
        for j in indices[indptr[i]:indptr[i + 1]]:
            cnt.setdefault((i // 16, int(j) // 16), []).append((i, int(j)))
    tiles = sorted(k for k, v in cnt.items() if len(v) >= min_nnz)
    masks = []
    for t in tiles:
        bits = 0
        for (i, j) in cnt[t]:
            bits |= 1 << ((i % 16) * 16 + (j % 16))
        masks.append([(bits >> (64 * w)) & ((1 << 64) - 1) for w in range(4)])
    tset = set(tiles)
    rows = [[int(j) for j in indices[indptr[i]:indptr[i + 1]] if (i // 16, int(j) // 16) not in tset]
            for i in range(n)]
    return tiles, masks, rows


@pytest.mark.parametrize("seed,n,min_nnz", [(0, 48, 192), (1, 70, 100), (2, 33, 1), (3, 16, 256)])
def test_tile_census_matches_brute_force(seed, n, min_nnz):
    rng = np.random.default_rng(200 + seed)
    a = rng.random((n, n)) < 0.08
    for b0 in range(0, n - 15, 16):                 # some dense blocks, some partial ones
        if rng.random() < 0.7:
            a[b0:b0 + 16, b0:b0 + 16] |= rng.random((16, 16)) < 0.9
    dst, src = np.nonzero(a)
    ip, ix = oracle.csr_build(src, dst, n)
    t = oracle.tile_census(ip, ix, n, min_nnz)
    tiles, masks, rows = _brute_tiles(ip, ix, n, min_nnz)
    assert [tuple(x) for x in t["tile_rc"].tolist()] == tiles
    assert t["tile_mask"].tolist() == masks
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    assert t["rindptr"].tolist() == rp.tolist()
    assert t["rindices"].tolist() == sum(rows, [])
    # invariants: popcounts + residual account for every edge once
    pop = sum(bin(int(w)).count("1") for w in t["tile_mask"].ravel())
    assert pop + t["rindices"].size == ix.size
    nb = (n + 15) // 16
    assert t["tile_ptr"].size == nb + 1 and t["tile_ptr"][-1] == len(tiles)
