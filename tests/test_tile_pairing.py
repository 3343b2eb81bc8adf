"""The B = 32 sweep's tile-list rule, modelled lane by lane on the CPU.

At B = 32 an exact 64-key tile holds two key blocks.  The sweep pairs key
blocks that the same query blocks of its group select (equal selection
masks), so both halves of a tile serve the same waves.  Wave 0 of a
workgroup builds the list: it scans key blocks in 64-block chunks in
ascending order; lane m (1 <= m < 2^nqb) keeps the state of selection mask
m, a block of that mask still waiting for a partner; in a chunk, the blocks
of mask m pair up in lane order, the first with the waiting one, and an odd
last one waits; the chunk's entries go out mask by mask; blocks left waiting
at the end get a tile of their own.

`build_tile_list` follows the kernel's arithmetic: the chunk's selection rows
as 64-bit words, each mask lane's set of blocks, its entry count, their
prefix over a row of 16 lanes, and per block the rank within its mask (a
population count below the lane) and its partner (the next lane of the same
mask), every entry written whole by one lane.  `plain_tile_list` states the
rule directly, mask by mask.  The tests check that the two agree entry for
entry, and the properties the sweep relies on, on random selections: every
selected key block in exactly one tile, paired blocks with equal masks,
entries dense from 0, and at most ceil(N / 2) + 8 entries (the list's LDS
size)."""
import numpy as np
import pytest

ALL = (1 << 64) - 1


def popc(x):
    return bin(x & ALL).count("1")


def build_tile_list(part, nqb, QB=4):
    """part[j]: selection mask of key block j over the group's nqb query
    blocks.  Returns {entry: (j1, j2 or None)} and the entry count."""
    N = len(part)
    all_blocks = (1 << nqb) - 1
    tiles, nt = {}, 0
    pend = [-1] * 64  # lane m: the waiting block of mask m
    for j0 in range(0, N, 64):
        # row b of the chunk: bit k for block j0 + k (blocks past N cleared)
        rowb = [sum(1 << k for k in range(64) if j0 + k < N and (part[j0 + k] >> b) & 1) for b in range(QB)]
        nz = 0
        for r in rowb:
            nz |= r
        lane_part = [sum(((rowb[b] >> l) & 1) << b for b in range(QB)) for l in range(64)]
        mine = []
        for l in range(64):
            m = nz
            for b in range(QB):
                m &= rowb[b] if (l >> b) & 1 else (~rowb[b] & ALL)
            mine.append(m if 1 <= l <= all_blocks else 0)
        c = [popc(m) for m in mine]
        q = [1 if c[l] > 0 and pend[l] >= 0 else 0 for l in range(64)]
        n = [q[l] + ((c[l] - q[l]) >> 1) if c[l] > 0 else 0 for l in range(64)]
        incl = [sum(n[16 * (l // 16): l + 1]) for l in range(64)]  # prefix within a row of 16 lanes
        first = [incl[l] - n[l] for l in range(64)]
        for l in range(64):
            pt = lane_part[l]
            if not pt:
                continue
            own, off, p = mine[pt], first[pt], pend[pt]
            qq = 1 if p >= 0 else 0
            r = popc(own & ((1 << l) - 1))
            above = own & ~((2 << l) - 1) & ALL
            if qq and r == 0:
                k, v = nt + off, (p, j0 + l)
            elif ((r - qq) & 1) == 0 and above:
                k, v = nt + off + qq + ((r - qq) >> 1), (j0 + l, j0 + (above & -above).bit_length() - 1)
            else:
                continue
            assert k not in tiles
            tiles[k] = v
        nt += incl[15]
        for l in range(64):
            if c[l] > 0:
                pend[l] = j0 + mine[l].bit_length() - 1 if (c[l] - q[l]) & 1 else -1
    waiting = [m for m in range(1, all_blocks + 1) if pend[m] >= 0]
    for i, m in enumerate(waiting):
        tiles[nt + i] = (pend[m], None)
    return tiles, nt + len(waiting)


def plain_tile_list(part, nqb):
    """The rule, mask by mask: in each 64-block chunk and for each mask in
    ascending order, the waiting block (if any) takes the chunk's first block
    of that mask, the rest pair up in order, an odd last one waits."""
    N = len(part)
    out, pend = [], {}
    for j0 in range(0, N, 64):
        for mk in range(1, 1 << nqb):
            blocks = [j for j in range(j0, min(N, j0 + 64)) if part[j] == mk]
            if not blocks:
                continue
            if mk in pend:
                out.append((pend.pop(mk), blocks[0]))
                blocks = blocks[1:]
            for i in range(0, len(blocks) - 1, 2):
                out.append((blocks[i], blocks[i + 1]))
            if len(blocks) % 2:
                pend[mk] = blocks[-1]
    out += [(pend[m], None) for m in sorted(pend)]
    return out


def random_parts(rng, nqb, N):
    sel = rng.random((nqb, N)) < rng.uniform(0, 1)
    if rng.random() < 0.4:  # rows that mostly agree, as neighbouring query blocks do
        sel[:] = sel[0] & (rng.random((nqb, N)) < 0.9)
    return [int(sum(int(sel[b, j]) << b for b in range(nqb))) for j in range(N)]


@pytest.mark.parametrize("seed", range(6))
def test_pairing_covers_the_union_with_equal_masks(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        nqb = int(rng.integers(1, 5))
        N = int(rng.integers(1, 600))
        part = random_parts(rng, nqb, N)
        tiles, nt = build_tile_list(part, nqb)
        assert sorted(tiles) == list(range(nt))
        assert [tiles[k] for k in range(nt)] == plain_tile_list(part, nqb)
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
    assert [tiles[k] for k in range(nt)] == plain_tile_list(part, nqb)
    singles = sum(1 for (j1, j2) in tiles.values() if j2 is None)
    assert singles <= (1 << nqb) - 1
