"""Host-side check of the streaming work split's invariant: no view is cut by two chunk boundaries.

The bf16 streaming attention lays each row block's views end to end in the order V-1, 0, V-2, 1, ...
and cuts the sequence into V equal chunks (chunk c = [floor(c*N/V), floor((c+1)*N/V)) of the N
tiles).  A view of the newest frames has a + b*u tiles for view u (a, b fixed per row block), so
each long/short pair fills exactly two chunks: the long view is cut once, the short one is whole,
and with V odd the middle view is one chunk.  The library relies on it (a view cut once is merged
in the attention kernel; a launch that found a second cut is refused).  This restates the split in
plain Python and checks the claim over a sweep of geometries.
"""
import itertools

import pytest


def view_tiles(P, T, F, qtok_end, u, TK=64):
    """Tiles of view u's key sequence for a row block whose last query token ends at qtok_end."""
    n_p = -(-P // TK)
    tps = -(-T // TK)
    ndiag = -(-qtok_end // TK)
    return n_p + (u * F + F - 1) * tps + ndiag


def cuts_per_view(V, F, T, P, G):
    HPW = G if G <= 2 else 4   # query heads per row block (a ragged last subset when 4 does not divide G)
    TBW = 4 // HPW
    nqb = -(-T // (32 * TBW))
    out = []
    for qb in range(nqb):
        end = min(T, (qb + 1) * 32 * TBW)
        tiles = [view_tiles(P, T, F, end, u) for u in range(V)]
        n = sum(tiles)
        bounds = [c * n // V for c in range(1, V)]   # the chunk boundaries strictly inside
        order = [(oi // 2) if oi % 2 else V - 1 - oi // 2 for oi in range(V)]
        pos = 0
        for u in order:
            out.append(sum(1 for b in bounds if pos < b < pos + tiles[u]))
            pos += tiles[u]
    return out


@pytest.mark.parametrize("V,F", list(itertools.product([2, 3, 4, 5, 6, 8], [1, 2, 4, 7, 8])))
def test_no_view_cut_twice(V, F):
    for T, P, G in itertools.product([1, 37, 64, 100, 256, 512], [0, 5, 64, 512, 700], [1, 2, 3, 4, 5, 6, 7, 8]):
        cuts = cuts_per_view(V, F, T, P, G)
        assert max(cuts) <= 1, (V, F, T, P, G, cuts)


def test_long_view_of_each_pair_cut_once():
    # config 3 of the workloads: 4 views, 4 frames, 256 tokens, prefix 512, G = 4: every row
    # block has two views cut once (the long one of each pair) and two whole
    cuts = cuts_per_view(4, 4, 256, 512, 4)
    assert len(cuts) == 8 * 4
    for qb in range(8):
        assert cuts[4 * qb: 4 * qb + 4] == [1, 0, 1, 0]
