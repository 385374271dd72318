"""The XCD-weighted deal of attention units to workgroup slots (pkv_decode_xcd_grid /
pkv_decode_xcd_slot_unit, host only): every unit in exactly one slot, each XCD's units in list
order, the even XCDs' share as asked, and bad arguments refused."""
import numpy as np
import pytest

import paged_kv_cache_306_amd as pkv

SPLITS = [0, 1, 100, 384, 500, 511, 512, 513, 538, 640, 1000, 1023]


def _deal(units, split):
    grid = pkv.decode_xcd_grid(units, split)
    return grid, np.array([pkv.decode_xcd_slot_unit(b, units, split) for b in range(grid)])


@pytest.mark.parametrize("units", [0, 1, 3, 8, 9, 40, 41, 320, 2560, 4640])
@pytest.mark.parametrize("split", SPLITS)
def test_every_unit_in_one_slot_in_list_order(units, split):
    grid, got = _deal(units, split)
    assert grid >= units and grid % (8 if split else 1) == 0
    assert np.array_equal(np.sort(got[got >= 0]), np.arange(units))
    assert np.all(got >= -1)
    for x in range(8):                      # workgroup b runs on XCD b % 8
        mine = got[x::8]
        mine = mine[mine >= 0]
        assert np.all(np.diff(mine) > 0)    # longest work first on every XCD
    if split == 0:
        assert np.array_equal(got, np.arange(units))


@pytest.mark.parametrize("split", [384, 450, 512, 538, 600, 640])
def test_even_share_follows_the_split(split):
    units = 5000
    _, got = _deal(units, split)
    even = np.zeros(units, bool)
    for b, u in enumerate(got):
        if u >= 0:
            even[u] = (b % 8) % 2 == 0
    # over every stretch of the list the even half takes split / 1024 of the units
    for lo in range(0, units, 500):
        assert abs(even[lo:lo + 500].mean() - split / 1024) <= 2 / 500
    # and the four XCDs of a half share its units evenly
    counts = [int(np.sum(got[x::8] >= 0)) for x in range(8)]
    assert max(counts[0::2]) - min(counts[0::2]) <= 1
    assert max(counts[1::2]) - min(counts[1::2]) <= 1


def test_grid_is_small():
    for split in (384, 640):
        assert pkv.decode_xcd_grid(100000, split) <= 1.25 * 100000 + 8


def test_bad_arguments():
    assert pkv.decode_xcd_grid(-1, 512) == -1
    assert pkv.decode_xcd_grid(10, -1) == -1
    assert pkv.decode_xcd_grid(10, 1024) == -1
    assert pkv.decode_xcd_slot_unit(-1, 10, 512) == -2
    assert pkv.decode_xcd_slot_unit(pkv.decode_xcd_grid(10, 600), 10, 600) == -2
    assert pkv.decode_xcd_slot_unit(0, 10, 1024) == -2
