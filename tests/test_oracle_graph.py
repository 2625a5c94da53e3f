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


def _brute_tiles(indptr, indices, n, min_nnz, T):
    nb = (n + 15) // 16
    deg = [indptr[i + 1] - indptr[i] for i in range(n)]
    odeg = [0] * n
    for j in indices:
        odeg[int(j)] += 1
    rb_ok = [all(deg[i] <= T for i in range(16 * b, min(n, 16 * b + 16))) for b in range(nb)]
    cb_ok = [all(odeg[j] <= T for j in range(16 * c, min(n, 16 * c + 16))) for c in range(nb)]
    seen = set()
    cand = {}                                   # pair -> list of CSR edge ids (first occurrences)
    for i in range(n):
        for e in range(indptr[i], indptr[i + 1]):
            j = int(indices[e])
            if (i, j) in seen:
                continue
            seen.add((i, j))
            if rb_ok[i // 16] and cb_ok[j // 16]:
                cand.setdefault((i // 16, j // 16), []).append(e)
    tiles = sorted(k for k, v in cand.items() if len(v) >= min_nnz)
    in_tile = set()
    masks = []
    for t in tiles:
        bits = 0
        for e in cand[t]:
            i = int(np.searchsorted(indptr, e, side="right") - 1)
            bits |= 1 << ((i % 16) * 16 + int(indices[e]) % 16)
            in_tile.add(e)
        masks.append([(bits >> (64 * w)) & ((1 << 64) - 1) for w in range(4)])
    rows = [[int(indices[e]) for e in range(indptr[i], indptr[i + 1]) if e not in in_tile] for i in range(n)]
    rb_t = [sum(1 for t in tiles if t[0] == b) for b in range(nb)]
    cb_t = [sum(1 for t in tiles if t[1] == c) for c in range(nb)]
    ctile = sorted(range(len(tiles)), key=lambda k: (tiles[k][1], tiles[k][0]))
    light_nt = [i for i in range(n) if deg[i] <= T and rb_t[i // 16] == 0]
    c_light_nt = [j for j in range(n) if odeg[j] <= T and cb_t[j // 16] == 0]
    return dict(tiles=tiles, masks=masks, rows=rows, rb_t=rb_t, cb_t=cb_t, ctile=ctile, light_nt=light_nt,
                c_light_nt=c_light_nt)


@pytest.mark.parametrize("seed,n,min_nnz,T", [(0, 48, 192, 10 ** 6), (1, 70, 100, 10 ** 6), (2, 33, 1, 10 ** 6),
                                              (3, 16, 256, 10 ** 6), (4, 64, 150, 18), (5, 80, 120, 25)])
def test_tile_census_matches_brute_force(seed, n, min_nnz, T):
    rng = np.random.default_rng(200 + seed)
    a = rng.random((n, n)) < 0.08
    for b0 in range(0, n - 15, 16):                 # some dense blocks, some partial ones
        if rng.random() < 0.7:
            a[b0:b0 + 16, b0:b0 + 16] |= rng.random((16, 16)) < 0.9
    dst, src = np.nonzero(a)
    ip, ix = oracle.csr_build(src, dst, n)
    t = oracle.tile_census(ip, ix, n, min_nnz, T)
    b = _brute_tiles(ip, ix, n, min_nnz, T)
    assert [tuple(x) for x in t["tile_rc"].tolist()] == b["tiles"]
    assert t["tile_mask"].tolist() == b["masks"]
    rp = np.concatenate([[0], np.cumsum([len(r) for r in b["rows"]])])
    assert t["rindptr"].tolist() == rp.tolist()
    assert t["rindices"].tolist() == sum(b["rows"], [])
    assert t["tile_ptr"].tolist() == np.concatenate([[0], np.cumsum(b["rb_t"])]).tolist()
    assert t["ctile_ptr"].tolist() == np.concatenate([[0], np.cumsum(b["cb_t"])]).tolist()
    assert t["ctile"].tolist() == b["ctile"]
    assert t["light_nt"].tolist() == b["light_nt"] and t["c_light_nt"].tolist() == b["c_light_nt"]
    assert t["trb"].tolist() == [k for k, v in enumerate(b["rb_t"]) if v]
    assert t["tcb"].tolist() == [k for k, v in enumerate(b["cb_t"]) if v]
    cip, cix = oracle.csc(t["rindptr"], t["rindices"], n)
    assert np.array_equal(t["rcindptr"], cip) and np.array_equal(t["rcindices"], cix)
    # invariants: popcounts + residual account for every edge once
    pop = sum(bin(int(w)).count("1") for w in t["tile_mask"].ravel())
    assert pop + t["rindices"].size == ix.size
    if T < 10 ** 6:
        deg = np.diff(ip)
        for rb, _ in t["tile_rc"]:
            assert np.all(deg[16 * rb:16 * rb + 16] <= T)


def test_tile_census_multigraph_copies_stay_residual():
    n = 16
    rows = [np.concatenate([np.arange(16), [3, 3]]) if i == 2 else np.arange(16) for i in range(n)]
    ip = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ix = np.concatenate(rows).astype(np.int32)
    t = oracle.tile_census(ip, ix, n, 256, 10 ** 6)
    assert t["tile_rc"].tolist() == [[0, 0]]
    assert all(int(w) == (1 << 64) - 1 for w in t["tile_mask"][0])
    assert t["rindices"].tolist() == [3, 3] and np.diff(t["rindptr"]).tolist()[2] == 2


def test_launch_order():
    indptr = np.array([0, 3, 3, 8, 10, 13, 14], np.int32)     # degrees 3, 0, 5, 2, 3, 1
    light = np.array([0, 1, 3, 4, 5], np.int32)
    assert oracle.launch_order(indptr, light, 1).tolist() == [0, 4, 3, 5, 1]
    assert oracle.launch_order(indptr, light, 0).tolist() == [0, 1, 3, 4, 5]
    # threshold 8 -> hoist degree > 2: degree 3 rows (ids 0, 4) first, the rest by id
    assert oracle.launch_order(indptr, light, 2, 8).tolist() == [0, 4, 1, 3, 5]
    ip = np.array([0, 1, 9, 14, 14, 30], np.int32)            # degrees 1, 8, 5, 0, 16
    assert oracle.launch_order(ip, np.arange(5), 2, 8).tolist() == [4, 1, 2, 0, 3]
    # order 3 (packed launches): descending ceil(degree / 4), ties by id.
    # degrees 7, 5, 8, 4, 1, 6, 0, 9: 4-edge steps 2, 2, 2, 1, 1, 2, 0, 3
    ip = np.concatenate([[0], np.cumsum([7, 5, 8, 4, 1, 6, 0, 9])]).astype(np.int32)
    assert oracle.launch_order(ip, np.arange(8), 3).tolist() == [7, 0, 1, 2, 5, 3, 4, 6]
    # strict descending degree would interleave the step-2 rows: 2, 0, 5, 1
    assert oracle.launch_order(ip, np.arange(8), 1).tolist() == [7, 2, 0, 5, 1, 3, 4, 6]
