"""CPU model of the balanced gather/scatter partition (no GPU).

A gather or scatter call with 16-byte aligned rows numbers its 16-byte units
row by row (row r: its state units, then its window units); workgroup w of G
takes units [U w / G, U (w + 1) / G) and walks the (row, region) pieces they
cover, each piece at most 2^27 units (one buffer resource).  The walk is
restated from `rows_balanced_kernel` (copy_kernels.hip); this checks that the
pieces of all workgroups cover every unit of every row exactly once, that a
piece never leaves its region of its row, and that the work per workgroup is
even.
"""
import numpy as np
import pytest

MAX_PIECE = 1 << 27
BLOCK_UNITS = 1024 * 8


def pieces(us, uw, n, G, w):
    upr = us + uw
    total = upr * n
    end = total * (w + 1) // G
    u = total * w // G
    out = []
    while u < end:
        row = u // upr
        ur = u - row * upr
        reg = 0 if ur < us else 1
        off = ur if reg == 0 else ur - us
        ln = min(end - u, (us if reg == 0 else uw) - off, MAX_PIECE)
        assert ln > 0
        out.append((row, reg, off, ln))
        u += ln
    return out


def grid_for(us, uw, n, resident):
    """Two resident rounds of workgroups, none with less than one block."""
    units = (us + uw) * n
    return max(1, min(2 * resident, -(-units // BLOCK_UNITS)))


@pytest.mark.parametrize("us,uw,n", [
    (2097152 // 16, 49152 // 16, 64),    # the 32-head geometry, 64 rows
    (2048 // 16, 384 // 16, 6),          # the tiny geometry
    (0, 96 // 16, 6),                    # a conv-window-only pool
    (2097152 // 16, 49152 // 16, 1),     # one row: fewer units than a grid
    (4096, 3, 1000),                     # many rows, tiny window
    (MAX_PIECE + 5, 1, 2),               # a region larger than one buffer resource
])
@pytest.mark.parametrize("resident", [1, 7, 512])
def test_partition_covers_every_unit_once(us, uw, n, resident):
    G = grid_for(us, uw, n, resident)
    seen = {}
    sizes = []
    for w in range(G):
        ps = pieces(us, uw, n, G, w)
        sizes.append(sum(p[3] for p in ps))
        for row, reg, off, ln in ps:
            assert 0 <= row < n
            assert 0 <= off and off + ln <= (us if reg == 0 else uw)
            assert ln <= MAX_PIECE
            seen.setdefault((row, reg), []).append((off, ln))
    for row in range(n):
        for reg, size in ((0, us), (1, uw)):
            iv = sorted(seen.get((row, reg), []))
            pos = 0
            for off, ln in iv:
                assert off == pos, "gap or overlap"
                pos += ln
            assert pos == size
    assert max(sizes) - min(sizes) <= 1, "uneven shares"
