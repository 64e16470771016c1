"""The persistent forward kernels' tile schedule, restated on the host.

Both forward kernels launch grid = min(G, C) workgroups, C the compute-unit
count rounded down to a multiple of 8, for G (b, h, query tile) tiles. In
pass r, workgroup w (on XCD x = w % 8, position b8 = w // 8 within it) takes
slot r*grid + 8*(b8 or g8-1-b8 on odd passes) + x, stops at the first slot
>= G, and renumbers the slot to a tile id so that each XCD's tiles are
consecutive ids. This checks that the walk visits every tile exactly once
and that no id leaves [0, G), for every G up to 2000 and several CU counts.
"""
import pytest


def schedule(G, cus):
    cap = cus & ~7
    grid = min(G, cap)
    per, rem = G >> 3, G & 7
    g8 = grid >> 3
    seen = []
    for w in range(grid):
        b8, x = w >> 3, w & 7
        r = 0
        while r * grid < G:
            slot = r * grid + 8 * ((g8 - 1 - b8) if (r & 1) else b8) + x
            if slot >= G:
                break
            assert slot >= 0
            seen.append((w, x * per + min(x, rem) + (slot >> 3)))
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
