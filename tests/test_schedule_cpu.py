"""The persistent pass's block schedule, checked by brute force on the CPU.

[FI] "Strategia di Tiling (Algoritmo 1)": after position i-1 the tile of side
U = lowbit(i) adds inputs [i-U, i) into outputs [i, i+U); every pair s < t is
covered once.  The persistent pass (k_run, T < 256) regroups the tiles of
side 256 and 512 into 256 x 256 block products: at a block boundary i with
i mod 1024 = o > 0 the next block [i, i+256) gets the products of the o/256
input blocks [i-o, i) ([FI] "Definizione di Aggregazione di Contribuzione":
a tile's contribution splits over any partition of its input and output
ranges).  Tiles of side < 256 are the in-register block triangle, sides
>= 1024 FFT tiles.  These tests restate those rules in plain Python and
check (1) that the regrouped schedule covers exactly the pairs the relaxed
tiling's tiles of side 256 and 512 cover, and (2) the rule by which a block
finds its successor's accumulators in the channel row: only FFT tiles (side
>= 1024) write the row, beyond their first 256 outputs; the first tile of a
level stores, later ones add.
"""
import numpy as np
import pytest

BLK, PERIOD = 256, 1024


def products(i):
    """Input block starts of the products at boundary i (the kernel's rule)."""
    o = i % PERIOD
    return [i - BLK * (p + 1) for p in range(o // BLK)]


@pytest.mark.parametrize("L", [700, 1000, 1024, 2048, 3000, 4096])
def test_block_products_cover_the_tiles_of_side_256_and_512(L):
    got = np.zeros((L, L), np.int8)
    for i in range(BLK, L, BLK):
        for tin in products(i):
            got[i:min(i + BLK, L), tin:tin + BLK] += 1
    want = np.zeros((L, L), np.int8)
    for i in range(1, L):
        U = i & -i
        if BLK <= U < PERIOD:
            want[i:min(i + U, L), i - U:i] += 1
    assert np.array_equal(got, want)


@pytest.mark.parametrize("L", [1000, 2048, 5000, 16384, 65536])
def test_row_holds_accumulators_exactly_where_the_rule_says(L):
    written = set()
    for i in range(1, L):
        U = i & -i
        if U < PERIOD:
            continue
        for p in range(i + BLK, min(i + U, L)):
            if i == U:      # first tile of its level: stores
                assert p not in written
                written.add(p)
            else:           # later tiles of the level add to a stored value
                assert p in written
    lp = PERIOD.bit_length() - 1
    for base in range(BLK, L, BLK):
        covered = any(j + BLK <= base < j + (j & -j) for j in range(PERIOD, base, PERIOD) if (j & -j) >= PERIOD)
        rule = ((base & (base - 1)) >> lp) != 0   # a set bit >= PERIOD other than the lowest
        assert covered == rule, base
