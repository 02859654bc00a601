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


# The block product's B operand, as the kernel addresses it (mm16_steps): a
# slot holds two reversed copies of the block's inputs, copy c holding x[p] at
# half 287 + c - p (zero padding elsewhere); in step n lane l reads the eight
# halves [m, m + 8) of copy cp, with r = l % 16, g = l // 16, d0 = 8 (g % 2),
# bh = g // 2, e0 = 287 - (r + 16 bh - d0), cp = e0 % 2, m = e0 + cp - 32 n.
def b_halves(n):
    out = set()
    for l in range(64):
        r, g = l & 15, l >> 4
        d0, bh = 8 * (g & 1), g >> 1
        e0 = 287 - (r + 16 * bh - d0)
        cp = e0 & 1
        m = e0 + cp - 32 * n
        assert m % 2 == 0 and 0 <= m and m + 8 <= 304
        out |= {(cp, m + j) for j in range(8)}
    return out


def inputs_of(halves):
    return {287 + c - m for c, m in halves if 0 <= 287 + c - m < BLK}


def test_product_steps_reach_inputs_in_order():
    """Step n of a block product reads inputs below 32 n + 32 and no others
    (step n pairs bt = 2n, 2n+1: x[a - d + 16 bt] with a, d < 16), so steps
    0 .. 3 need only the block's first 128 inputs: the closed loop forms them
    during the chain, once those inputs are final."""
    for n in range(9):
        got = inputs_of(b_halves(n))
        assert max(got) == min(32 * n + 31, BLK - 1), n
    assert max(inputs_of(set().union(*(b_halves(n) for n in range(4))))) == 127
    assert min(inputs_of(b_halves(4))) < 128 <= max(inputs_of(b_halves(4)))


def test_early_steps_and_late_inputs_touch_disjoint_halves():
    """While the other wavefront reads the halves of steps 0 .. 3 (and writes
    the fp16 parts of inputs below 128), the chain wavefront writes those of
    inputs 128 .. 255 into the same slot: the two sets of halves must not
    meet, in either copy."""
    early = set().union(*(b_halves(n) for n in range(4)))
    first = {(0, 287 - p) for p in range(128)} | {(1, 288 - p) for p in range(128)}
    late = {(0, 287 - p) for p in range(128, BLK)} | {(1, 288 - p) for p in range(128, BLK)}
    assert not early & late
    assert not first & late
    # every input half that steps 0 .. 3 read is one the other wavefront wrote
    assert {h for h in early if 0 <= 287 + h[0] - h[1] < BLK} <= first
