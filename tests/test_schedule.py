"""The persistent tile schedule (`persistent_tile` in fmha_fwd_kernel.hpp),
restated on the host.

Both forward kernels launch grid = min(G, C) workgroups, C the compute-unit
count rounded down to a multiple of 8, for G tiles. Each workgroup asks for pass r = 0, 1, ... until the answer is -1: no
pass r when r*grid >= G; otherwise workgroup w (on XCD x = w % 8, position
b8 = w // 8 within it) takes slot r*grid + 8*(b8 or g8-1-b8 on odd passes) +
x, none when that slot is >= G, and the slot is renumbered to a tile id so
that each XCD's tiles are consecutive ids. This checks that the walk visits
every tile exactly once and that no id leaves [0, G), for every G up to 2000
and several CU counts.
"""
import pytest


def persistent_tile(r, G, grid, w):
    """The kernel's function, line for line in meaning."""
    if r * grid >= G:
        return -1
    g8, b8, x = grid >> 3, w >> 3, w & 7
    slot = r * grid + 8 * ((g8 - 1 - b8) if (r & 1) else b8) + x
    if slot >= G:
        return -1
    per, rem = G >> 3, G & 7
    return x * per + min(x, rem) + (slot >> 3)


def schedule(G, cus):
    """(workgroup, tile) pairs as the kernels walk them: each workgroup
    stops at its first pass without a tile."""
    grid = min(G, cus & ~7)
    seen = []
    for w in range(grid):
        r = 0
        while True:
            t = persistent_tile(r, G, grid, w)
            if t < 0:
                break
            seen.append((w, t))
            r += 1
    return grid, seen


@pytest.mark.parametrize("cus", [256, 304, 80, 8, 15])
def test_every_tile_once(cus):
    for G in range(1, 2001):
        grid, seen = schedule(G, cus)
        ids = sorted(t for _, t in seen)
        assert ids == list(range(G)), (G, cus)


def test_work_per_workgroup_is_balanced():
    """Whole passes give each workgroup the same number of tiles; a partial
    last pass adds at most one."""
    for G in (8192, 512, 1000, 372, 257):
        grid, seen = schedule(G, 256)
        counts = [0] * grid
        for w, _ in seen:
            counts[w] += 1
        assert max(counts) - min(counts) <= 1 and sum(counts) == G


def test_each_xcd_holds_consecutive_ids():
    """Within one pass the tiles an XCD receives are consecutive ids, so the
    query tiles of one head share that XCD's L2."""
    G, grid = 8192, 256
    _, seen = schedule(G, grid)
    by_x = {}
    for w, t in seen:
        by_x.setdefault(w & 7, []).append(t)
    for x, ids in by_x.items():
        ids.sort()
        assert ids == list(range(ids[0], ids[0] + len(ids))), x


def test_one_workgroup_per_tile_gets_no_second_pass():
    """With as many workgroups as tiles and G not a multiple of 8, the odd
    pass's reversed walk lands below G (8 * (g8 - 1 - b8) < 0 for the last,
    partial group of 8); the schedule must end after pass 0. An earlier walk
    without the r * grid >= G test took any slot below G, negative ones
    included, and so handed some workgroups a second copy of a tile already
    taken (2 at G = 3, 6 at G = 7, 4 at G = 12 and at G = 100, 7 at G = 255)."""
    for G, dups in ((3, 2), (7, 6), (12, 4), (100, 4), (255, 7)):
        grid, seen = schedule(G, 256)
        assert grid == G
        assert sorted(w for w, _ in seen) == list(range(G)), G

        def old_pass1(w):
            g8, b8, x = grid >> 3, w >> 3, w & 7
            slot = grid + 8 * (g8 - 1 - b8) + x
            per, rem = G >> 3, G & 7
            return x * per + min(x, rem) + (slot >> 3) if slot < G else -1
        assert sum(old_pass1(w) >= 0 for w in range(grid)) == dups, G
