"""CPU model of the gradient tiles' transposed W chunk (no GPU needed).

lce_backward's dZ tiles also write W's chunk transposed, WT[k][c - c0], from the W rows
they stage through LDS: stage s of the K loop belongs to the tile whose row tile is
s % n_row_tiles.  The write uses ds_read_b64_tr_b16, whose lane layout was taken from a
probe on the GPU: within each 16-lane group, output lane j's element e is element j % 4
of the 8 bytes that lane j // 4 + 4 e addresses.  This model replays the kernel's
addressing (the XOR-swizzled stage layout, the clamped rows past the chunk, the zero K
tail) and checks that every LDS address stays inside the stage's W tile and that every
element of WT[:, :w8] is written exactly once, with W's value or, past the chunk's w
columns, zero.
"""

import numpy as np
import pytest

BN, BK = 256, 64


def tr_read(addrs, lds_value):
    """ds_read_b64_tr_b16 on one 16-lane group."""
    m = [[lds_value(a + 2 * e) for e in range(4)] for a in addrs]
    return [[m[(j >> 2) + 4 * e][j & 3] for e in range(4)] for j in range(16)]


def swizzled(row, kk):
    """Byte offset of K values kk .. kk + 3 of tile row `row` (kk a multiple of 4)."""
    return row * 128 + (((kk >> 3) ^ ((row >> 1) & 7)) << 4) + (kk & 7) * 2


def model(N, D, W, c0, width, ld, offset=swizzled):
    n_row_tiles = (N + BN - 1) // BN
    n_col_tiles = (width + BN - 1) // BN
    nk = (D + BK - 1) // BK
    c_end = c0 + width
    w8 = (width + 7) // 8 * 8
    WT = np.full((D, ld), -1, dtype=np.int64)
    count = np.zeros((D, ld), dtype=np.int64)
    for r in range(n_row_tiles):
        for cc in range(n_col_tiles):
            col0 = c0 + cc * BN
            b_rows = min(BN, c_end - col0)
            for s in range(nk):
                if s % n_row_tiles != r:
                    continue

                def lds_value(byte):
                    # the stage's W tile: row R holds W row col0 + R (clamped to the last
                    # valid row), 8 swizzled 16-byte chunks of K, zero past D
                    assert 0 <= byte < BN * 128 and byte % 2 == 0, byte
                    R = byte // 128
                    chunk = ((byte % 128) // 16) ^ ((R >> 1) & 7)
                    k = s * BK + chunk * 8 + (byte % 16) // 2
                    return int(W[min(col0 + R, col0 + b_rows - 1), k]) if k < D else 0

                for wave in range(4):
                    for it in range(8):
                        kb = 16 * (it >> 1)
                        for g in range(4):
                            cb = wave * 64 + 32 * (it & 1) + 8 * g
                            lo = tr_read([offset(cb + (j >> 2), kb + 4 * (j & 3)) for j in range(16)], lds_value)
                            hi = tr_read([offset(cb + 4 + (j >> 2), kb + 4 * (j & 3)) for j in range(16)], lds_value)
                            for j in range(16):
                                k = s * BK + kb + j
                                col = col0 + cb - c0
                                if k < D and col < w8:
                                    vals = lo[j] + hi[j]
                                    for t in range(8):
                                        WT[k, col + t] = vals[t] if c0 + col + t < c_end else 0
                                        count[k, col + t] += 1
    return WT, count, w8


def check(N, D, V, c0, width, ld, offset=swizzled):
    W = np.random.default_rng([N, D, V]).integers(1, 30000, size=(V, D))
    WT, count, w8 = model(N, D, W, c0, width, ld, offset)
    ref = np.zeros((D, w8), dtype=np.int64)
    ref[:, :width] = W[c0:c0 + width].T
    assert (count[:, :w8] == 1).all(), "an element of WT is written more than once or not at all"
    assert (count[:, w8:] == 0).all(), "a write past the padded chunk width"
    assert (WT[:, :w8] == ref).all(), "a wrong value in WT"


@pytest.mark.parametrize("N,D,V,c0,width,ld", [
    (1, 8, 1, 0, 1, 256),            # one row, one column, a K tail of 8
    (37, 40, 127, 0, 127, 256),      # one stage, chunk width not a multiple of 8
    (300, 72, 1000, 0, 1000, 1024),  # two row tiles, a K tail
    (600, 200, 700, 0, 700, 768),    # three row tiles, four stages
    (513, 128, 8193, 8192, 1, 8192), # the one-column last chunk of 8193
])
def test_every_element_written_once_with_its_value(N, D, V, c0, width, ld):
    check(N, D, V, c0, width, ld)


def test_model_catches_a_wrong_swizzle():
    """The checker itself: addressing the stage without its XOR swizzle must fail."""
    plain = lambda row, kk: row * 128 + kk * 2
    with pytest.raises(AssertionError):
        check(300, 72, 1000, 0, 1000, 1024, offset=plain)
