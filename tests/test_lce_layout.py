"""CPU model of lce_tile's global->LDS load addressing (no GPU needed).

lce_tile loads each 256-row tile of H (or W) in 64-column K stages: wave w, load group
q and lane l fetch 16 bytes for LDS row w*64 + q*8 + l/8, physical 16-byte chunk l % 8,
from the logical K chunk (l % 8) ^ ((row >> 1) & 7).  Rows past the matrix re-read its
last row; K chunks past D re-read the row's last chunk.  The address is a tile base
plus an unsigned 32-bit lane offset, which the hardware zero-extends.  This test
re-derives those addresses and checks that (1) every byte read lies inside the matrix,
(2) the 32-bit lane offset never wraps, and (3) the loads of one stage cover every
(row, K chunk) of the tile exactly once, which is what the fragment reads rely on.
"""

import numpy as np
import pytest

BM = 256
BK = 64


def koff():
    lanes = np.arange(64)
    out = np.zeros((2, 64), np.int64)
    for par in range(2):
        r = par * 8 + (lanes >> 3)
        out[par] = ((lanes & 7) ^ ((r >> 1) & 7)) * 8
    return out


def stage_loads(total_rows, D, tile, kt):
    """(byte offsets, 32-bit lane offsets, (row, logical chunk) pairs) of one stage."""
    lanes = np.arange(64)
    ko = koff()
    row0 = tile * BM
    nrows = min(total_rows - row0, BM)
    k0 = kt * BK
    offs, lane32, cover = [], [], []
    for w in range(4):
        lrow = w * 64 + (lanes >> 3)
        for q in range(8):
            r = lrow + q * 8
            rr = np.where(r < nrows, r, nrows - 1)
            kk = np.where(k0 + ko[q & 1] < D, ko[q & 1], D - 8 - k0)
            off32 = rr * D * 2 + kk * 2
            lane32.append(off32)
            offs.append(row0 * D * 2 + k0 * 2 + off32)
            # LDS slot (row r, physical chunk lane % 8) holds logical chunk ko / 8
            cover.append(np.stack([r, ko[q & 1] // 8, lanes & 7], axis=1))
    return np.concatenate(offs), np.concatenate(lane32), np.concatenate(cover)


SHAPES = [(1, 8), (3, 8), (37, 40), (300, 72), (257, 520), (513, 128), (255, 200), (64, 4096)]


@pytest.mark.parametrize("rows,D", SHAPES)
def test_loads_stay_inside_the_matrix(rows, D):
    n_tiles = (rows + BM - 1) // BM
    for t in range(n_tiles):
        for kt in range((D + BK - 1) // BK):
            off, lane32, _ = stage_loads(rows, D, t, kt)
            assert lane32.min() >= 0 and lane32.max() < 2 ** 32
            assert off.min() >= 0
            assert off.max() + 16 <= rows * D * 2


def test_full_size_tiles_stay_inside():
    for rows in (8192, 151936):
        n_tiles = (rows + BM - 1) // BM
        for t in (0, 1, n_tiles // 2, n_tiles - 1):
            for kt in (0, 1, 63):
                off, lane32, _ = stage_loads(rows, 4096, t, kt)
                assert lane32.max() < 2 ** 32 and off.min() >= 0 and off.max() + 16 <= rows * 4096 * 2


def test_one_stage_covers_each_row_chunk_once():
    _, _, cover = stage_loads(1024, 4096, 1, 5)
    rows, logical, physical = cover[:, 0], cover[:, 1], cover[:, 2]
    assert len(cover) == BM * 8
    pairs = set(zip(rows.tolist(), logical.tolist()))
    assert pairs == {(r, c) for r in range(BM) for c in range(8)}
    # and the swizzle maps each row's 8 logical chunks to its 8 physical slots
    assert np.all(physical == (logical ^ ((rows >> 1) & 7)))


def test_fragment_reads_are_bank_spread():
    """The 16 rows an MFMA operand read touches at one K chunk use 16 distinct
    16-byte slots within a 256-byte LDS window."""
    for c in range(8):
        rows = np.arange(16)
        byte = rows * 128 + ((c ^ ((rows >> 1) & 7)) << 4)
        assert len(set((byte % 256 // 16).tolist())) == 16
