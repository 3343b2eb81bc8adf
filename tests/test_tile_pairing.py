"""The B = 32 sweep's tile-list rule, modelled lane by lane on the CPU.

At B = 32 an exact 64-key tile holds two key blocks.  The sweep pairs key
blocks that the same query blocks of its group select (equal selection
masks), so both halves of a tile serve the same waves.  Wave 0 of a
workgroup builds the list: it scans key blocks in 64-block chunks in
ascending order; lane m of a register holds a block of mask m still waiting
for a partner; in a chunk, the blocks of mask m pair up in lane order, the
first with the waiting one, and an odd last one waits; blocks left waiting at
the end get a tile of their own.  This model follows the kernel's arithmetic
(ranks by population count of a ballot, entry index nt + q + (r - q) / 2,
the first half stored before the second is merged in) and checks the
properties the sweep relies on, on random selections: every selected key
block in exactly one tile, paired blocks with equal masks, entries dense
from 0, and at most ceil(N / 2) + 8 entries (the list's LDS size)."""
import numpy as np
import pytest


def build_tile_list(part, nqb):
    """part[j]: selection mask of key block j over the group's nqb query
    blocks.  Returns {entry: (j1, j2 or None)} and the entry count."""
    N = len(part)
    all_blocks = (1 << nqb) - 1
    tiles, nt = {}, 0
    pend = [-1] * 64
    for j0 in range(0, N, 64):
        lane_j = [j0 + l for l in range(64)]
        lane_part = [part[j] if j < N else 0 for j in lane_j]
        for mk in range(1, all_blocks + 1):
            lanes = [l for l in range(64) if lane_part[l] == mk]  # the ballot, in lane order
            if not lanes:
                continue
            c, p = len(lanes), pend[mk]
            q = 1 if p >= 0 else 0
            first = {}
            for r, l in enumerate(lanes):
                if q and r == 0:
                    first[nt] = (p, lane_j[l])
                elif ((r - q) & 1) == 0 and r + 1 < c:
                    first[nt + q + ((r - q) >> 1)] = (lane_j[l], None)
            for k, v in first.items():
                assert k not in tiles
                tiles[k] = v
            for r, l in enumerate(lanes):
                if r >= q and ((r - q) & 1) == 1:
                    k = nt + q + ((r - q) >> 1)
                    assert tiles[k][1] is None
                    tiles[k] = (tiles[k][0], lane_j[l])
            rest = c - q
            nt += q + (rest >> 1)
            pend[mk] = lane_j[lanes[-1]] if rest & 1 else -1
    waiting = [m for m in range(1, all_blocks + 1) if pend[m] >= 0]
    for i, m in enumerate(waiting):
        tiles[nt + i] = (pend[m], None)
    return tiles, nt + len(waiting)


@pytest.mark.parametrize("seed", range(6))
def test_pairing_covers_the_union_with_equal_masks(seed):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        nqb = int(rng.integers(1, 5))
        N = int(rng.integers(1, 600))
        sel = rng.random((nqb, N)) < rng.uniform(0, 1)
        part = [int(sum(int(sel[b, j]) << b for b in range(nqb))) for j in range(N)]
        tiles, nt = build_tile_list(part, nqb)
        assert sorted(tiles) == list(range(nt))
        seen = []
        for k in range(nt):
            j1, j2 = tiles[k]
            seen.append(j1)
            if j2 is not None:
                seen.append(j2)
                assert j1 < j2 and part[j1] == part[j2]
        assert sorted(seen) == [j for j in range(N) if part[j]]
        assert nt <= (N + 1) // 2 + 8


def test_pairing_wastes_at_most_one_half_per_mask():
    """Halves a wave computes without having selected them: only the
    unpaired blocks, at most one per selection mask."""
    rng = np.random.default_rng(7)
    nqb, N = 4, 4096
    sel = rng.random((nqb, N)) < 0.1
    part = [int(sum(int(sel[b, j]) << b for b in range(nqb))) for j in range(N)]
    tiles, nt = build_tile_list(part, nqb)
    singles = sum(1 for (j1, j2) in tiles.values() if j2 is None)
    assert singles <= (1 << nqb) - 1
