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


# ---- the measurement the step driver makes from one stamped launch (host only)

def _launch(units, speed_even, speed_odd, seed=0, slots_per_xcd=96, tail_boost=1.0):
    """Stamps of a simulated launch dealing unit b to workgroup b (XCD b % 8): each XCD runs its
    units in order on `slots_per_xcd` slots at its half's tokens per tick; once the first XCD
    has no work left, the others run `tail_boost` times faster (they share its bandwidth)."""
    g = np.random.default_rng(seed)
    tokens = np.sort(g.integers(128, 2049, units))[::-1]
    start = np.zeros(units)
    end = np.zeros(units)
    for x in range(8):
        free = np.zeros(slots_per_xcd)
        for b in range(x, units, 8):
            i = int(np.argmin(free))
            speed = speed_even if x % 2 == 0 else speed_odd
            start[b] = free[i]
            end[b] = free[i] + tokens[b] / speed
            free[i] = end[b]
    first_idle = min(end[x::8].max() for x in range(8))
    late = end > first_idle          # the part past the first XCD's end runs faster
    end[late] = first_idle + (end[late] - np.maximum(start[late], first_idle)) / tail_boost + \
        np.maximum(0, first_idle - start[late])
    st = np.zeros((units, 4), np.uint32)
    base = 123456789                 # arbitrary start tick, 32-bit wrap-safe
    st[:, 0] = np.maximum(1, np.round(end - start)).astype(np.uint32)
    st[:, 1] = 0x100 | (np.arange(units) % 8)
    st[:, 2] = tokens
    st[:, 3] = (base + np.round(start).astype(np.int64)) % (1 << 32)
    return st


def test_measured_split_follows_the_halves_speeds():
    for even, odd in [(1.0, 0.9), (1.0, 0.8), (0.9, 1.0)]:
        p, re_, ro, outcome = pkv.xcd_split_from_stamps(_launch(2560, even, odd))
        assert outcome == pkv.PKV_XCD_MEASURED
        assert abs(re_ / ro - even / odd) < 0.02
        assert abs(p - round(1024 * even / (even + odd))) <= 3


def test_workgroups_after_the_first_xcd_ends_are_left_out():
    # in the tail the remaining XCDs run faster; counting them would understate the gap
    p_all_fast, _, _, _ = pkv.xcd_split_from_stamps(_launch(2560, 1.0, 0.9, tail_boost=3.0))
    p_plain, _, _, _ = pkv.xcd_split_from_stamps(_launch(2560, 1.0, 0.9))
    assert abs(p_all_fast - p_plain) <= 3
    assert p_plain > 530


def test_equal_halves_keep_the_even_deal():
    p, re_, ro, outcome = pkv.xcd_split_from_stamps(_launch(2560, 1.0, 1.0))
    assert (p, outcome) == (0, pkv.PKV_XCD_MEASURED) and abs(re_ / ro - 1) < 0.01


def test_split_is_bounded():
    # 2:1 would ask for 683 / 341 of 1024
    p, _, _, outcome = pkv.xcd_split_from_stamps(_launch(2560, 1.0, 0.5))
    assert outcome == pkv.PKV_XCD_MEASURED and p == 640
    p, _, _, outcome = pkv.xcd_split_from_stamps(_launch(2560, 0.5, 1.0))
    assert outcome == pkv.PKV_XCD_MEASURED and p == 384


def test_unexpected_xcd_placement_turns_weighting_off():
    st = _launch(2560, 1.0, 0.9)
    st[17, 1] = 0x100 | 3                    # workgroup 17 reported on XCD 3, not 1
    p, _, _, outcome = pkv.xcd_split_from_stamps(st)
    assert (p, outcome) == (0, pkv.PKV_XCD_UNMAPPED)


def test_too_few_workgroups_cannot_tell():
    st = _launch(2560, 1.0, 0.9)
    st[200:, 1] = 0                          # only 200 workgroups attended tokens
    p, _, _, outcome = pkv.xcd_split_from_stamps(st)
    assert (p, outcome) == (-1, pkv.PKV_XCD_TOO_FEW)
    assert pkv.lib().pkv_xcd_split_from_stamps(None, 4, None, None, None) == -2
