"""CPU model of how the persistent kernels hand out output tiles, restated
from their index arithmetic:

* workgroup wg of nwg starts at tile (wg % 8) * (nwg / 8) + wg / 8 when nwg
  is a multiple of 8 (the dispatcher deals workgroups to the 8 XCDs round
  robin, so the workgroups of one XCD take one contiguous run of tile ids),
  else at tile wg; it then steps by nwg until it passes the last tile;
* a linear tile id becomes (tile row, tile column) in groups of group_m tile
  rows, column-major inside a group (tile_coords);
* a grouped GEMM lays its groups' tiles end to end; a tile finds its group
  by a binary search over the first-tile table (empty groups have equal
  neighbours) and its rows and column there (tile_ref).

Every output tile must be computed exactly once, whatever the grid."""
import itertools

import numpy as np
import pytest


def first_tile(wg, nwg):
    return (wg & 7) * (nwg >> 3) + (wg >> 3) if (nwg & 7) == 0 else wg


def schedule(ntiles, nwg):
    """tile ids each workgroup computes, in order"""
    out = []
    for wg in range(nwg):
        t, mine = first_tile(wg, nwg), []
        while t < ntiles:
            mine.append(t)
            t += nwg
        out.append(mine)
    return out


def tile_coords(tile, tiles_m, tiles_n, group_m):
    per_group = group_m * tiles_n
    g = tile // per_group
    first = g * group_m
    rows = min(tiles_m - first, group_m)
    idx = tile - g * per_group
    return first + idx % rows, idx // rows


def group_of(tile, gtiles):
    lo, hi = 0, len(gtiles) - 1
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if gtiles[mid] <= tile:
            lo = mid
        else:
            hi = mid
    return lo


@pytest.mark.parametrize("ntiles,nwg", [(1024, 256), (1000, 256), (81, 81), (260, 256), (7, 7), (300, 100),
                                        (313, 256), (64, 64), (4096, 256)])
def test_every_tile_once(ntiles, nwg):
    done = list(itertools.chain.from_iterable(schedule(ntiles, nwg)))
    assert sorted(done) == list(range(ntiles))


@pytest.mark.parametrize("ntiles,nwg", [(1024, 256), (1000, 256), (4096, 256), (64, 64)])
def test_xcd_runs_are_contiguous(ntiles, nwg):
    """In every round the 8 XCDs' workgroups take 8 contiguous runs of nwg / 8
    tile ids (so neighbouring tiles, which share operand panels, meet in one
    XCD's L2)."""
    per = nwg // 8
    for r in range(-(-ntiles // nwg)):
        for x in range(8):
            ids = sorted(r * nwg + first_tile(wg, nwg) for wg in range(x, nwg, 8))
            assert ids == list(range(r * nwg + x * per, r * nwg + (x + 1) * per))


@pytest.mark.parametrize("tiles_m,tiles_n,group_m", [(32, 32, 4), (9, 11, 4), (1, 64, 4), (13, 5, 4), (3, 7, 8),
                                                     (5, 1, 4)])
def test_tile_coords_is_a_bijection(tiles_m, tiles_n, group_m):
    seen = [tile_coords(t, tiles_m, tiles_n, group_m) for t in range(tiles_m * tiles_n)]
    assert sorted(seen) == [(m, n) for m in range(tiles_m) for n in range(tiles_n)]
    # column-major inside a group of tile rows: consecutive ids walk down the group's rows first
    for t in range(tiles_m * tiles_n - 1):
        (m0, n0), (m1, n1) = seen[t], seen[t + 1]
        if n1 == n0:
            assert m1 == m0 + 1
        elif m1 // group_m == m0 // group_m:
            assert n1 == n0 + 1 and m1 == (m0 // group_m) * group_m


@pytest.mark.parametrize("seed", range(6))
def test_grouped_tiles_cover_each_group_once(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.integers(1, 9))
    rows = rng.integers(0, 700, G)
    rows[rng.random(G) < 0.3] = 0                           # empty groups
    N, TM, TN = int(rng.integers(1, 900)), 256, int(rng.choice([64, 256]))
    goff = np.concatenate([[0], np.cumsum(rows)])
    tn = -(-N // TN)
    gtiles = np.concatenate([[0], np.cumsum([-(-r // TM) * tn for r in rows])])
    seen = set()
    for tile in range(int(gtiles[-1])):
        g = group_of(tile, list(gtiles))
        assert gtiles[g] <= tile < gtiles[g + 1] and rows[g] > 0
        tmg = -(-int(rows[g]) // TM)
        local = tile - gtiles[g]
        m0, n0 = goff[g] + (local % tmg) * TM, (local // tmg) * TN
        assert goff[g] <= m0 < goff[g + 1] and 0 <= n0 < N
        seen.add((g, int(m0), int(n0)))
    want = {(g, int(goff[g] + i * TM), j * TN) for g in range(G) for i in range(-(-int(rows[g]) // TM))
            for j in range(tn)}
    assert seen == want
