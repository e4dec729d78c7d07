"""Host check of the persistent flash-prefill work map (prefill_fast.hip,
prefill_flash_persist_kernel and its launcher): every (sequence, head, query tile) item runs
exactly once, and with an even number of query tiles every workgroup gets the same work.

The kernel's index arithmetic is restated here in Python (slot s of XCD x is item 8 s + x;
slot ntq j + r of an XCD is query tile ntq - 1 - r of its group j), so a change to either
side that breaks the map fails this test on the CPU."""
import pytest


def launch(B, H, ntq, cus=256):
    """Grid of the persistent form, or None when the launcher takes one workgroup per item."""
    n_items = ntq * H * B
    per = ntq // 2 if ntq % 2 == 0 else ntq
    cpx = (cus // 8) // per * per
    if (B * H) % 8 == 0 and cpx > 0 and n_items > 8 * cpx:
        return 8 * cpx, n_items
    return None, n_items


def walk(grid, n_items, ntq):
    """Items each workgroup runs, in order."""
    cpx = grid >> 3
    n_slots = n_items >> 3
    runs = []
    for w in range(grid):
        x, c = w & 7, w >> 3
        mine = []
        if ntq % 2 == 0:
            hq = ntq >> 1
            n_groups = n_slots // ntq
            gpr, t = cpx // hq, c % hq
            g = c // hq
            while g < n_groups:
                mine.append((g * ntq + t) * 8 + x)
                mine.append((g * ntq + ntq - 1 - t) * 8 + x)
                g += gpr
        else:
            jbase, jq = (c // ntq) * ntq, c % ntq
            k = 0
            while True:
                slot = cpx * k + jbase + (jq + k) % ntq
                if slot >= n_slots:
                    break
                mine.append(slot * 8 + x)
                k += 1
        runs.append(mine)
    return runs


def tile_of(L, ntq):
    """Query tile of item L (the kernel's map for group counts divisible by 8)."""
    slot = L >> 3
    return ntq - 1 - slot % ntq


@pytest.mark.parametrize("B,H,ntq", [(4, 128, 16), (2, 128, 2), (2, 128, 3), (4, 128, 4), (1, 64, 16),
                                     (4, 128, 5), (3, 64, 6), (8, 128, 1), (8, 16, 32), (1, 8, 16)])
def test_every_item_once(B, H, ntq):
    grid, n_items = launch(B, H, ntq)
    if grid is None:
        pytest.skip("one workgroup per item for this shape")
    runs = walk(grid, n_items, ntq)
    seen = sorted(L for r in runs for L in r)
    assert seen == list(range(n_items))


@pytest.mark.parametrize("B,H,ntq", [(4, 128, 16), (4, 128, 4), (3, 64, 6)])
def test_pairs_balance(B, H, ntq):
    """Each pair of tiles t, ntq-1-t costs ntq+1 tile lengths: equal work per workgroup when the
    groups divide evenly over the rounds."""
    grid, n_items = launch(B, H, ntq)
    runs = walk(grid, n_items, ntq)
    work = {sum(tile_of(L, ntq) + 1 for L in r) for r in runs}
    cpx, hq = grid >> 3, ntq // 2
    if (n_items // 8 // ntq) % (cpx // hq) == 0:
        assert len(work) == 1
    assert all(len(r) % 2 == 0 for r in runs)
