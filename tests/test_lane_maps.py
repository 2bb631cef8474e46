"""Lane algebra of the group-parameter reduce-scatters (host model, no GPU).

The fake quantisation (groups of 16 lanes) and the packing (groups of 8
lanes) reduce four rows' partial min / max so that each lane ends with the
group-wide values of one row, form that row's parameters, and broadcast them
back per row with ds_swizzle.  This models the cross-lane operations with
their documented lane maps (DPP row_mirror and row_half_mirror inside rows of
16 lanes, quad_perm inside quads, ds_swizzle's bitmask mode inside 32 lanes)
and checks, over a whole 64-lane wave, that

* after the reduce-scatter lane j holds exactly the min and max over its group
  of row (j >> 2) & 3 (16-lane groups) or (j >> 1) & 3 (8-lane groups), and
* the broadcast of row p reads a lane of the lane's own group that holds row p.

A wrong mirror, a swapped keep / send select or a wrong swizzle mask makes a
lane end with another row, or with a min over part of its group only.
"""

import numpy as np
import pytest

LANES = 64


def row_mirror(v):          # DPP row_mirror: lane i of a 16-lane row reads lane 15 - i
    return np.array([v[(i & ~15) | (15 - (i & 15))] for i in range(LANES)])


def row_half_mirror(v):     # DPP row_half_mirror: lane i of an 8-lane half-row reads 7 - i
    return np.array([v[(i & ~7) | (7 - (i & 7))] for i in range(LANES)])


def quad_perm(v, perm):     # DPP quad_perm: lane i of a quad reads lane perm[i % 4]
    return np.array([v[(i & ~3) | perm[i & 3]] for i in range(LANES)])


def swizzle_bitmask(v, and_mask, or_mask, xor_mask=0):
    """ds_swizzle bitmask mode: within each 32-lane half, lane i reads lane
    ((i & and_mask) | or_mask) ^ xor_mask."""
    return np.array([v[(i & 32) | (((i & 31) & and_mask) | or_mask) ^ xor_mask]
                     for i in range(LANES)])


def scatter4_16(mn, mx):
    """minmax_scatter4: four rows over groups of 16 lanes."""
    lane = np.arange(LANES)
    b3, b2 = (lane & 8) != 0, (lane & 4) != 0
    kn, kx = [], []
    for i in range(2):
        keep_n, send_n = np.where(b3, mn[2 + i], mn[i]), np.where(b3, mn[i], mn[2 + i])
        keep_x, send_x = np.where(b3, mx[2 + i], mx[i]), np.where(b3, mx[i], mx[2 + i])
        kn.append(np.minimum(keep_n, row_mirror(send_n)))
        kx.append(np.maximum(keep_x, row_mirror(send_x)))
    keep_n, send_n = np.where(b2, kn[1], kn[0]), np.where(b2, kn[0], kn[1])
    keep_x, send_x = np.where(b2, kx[1], kx[0]), np.where(b2, kx[0], kx[1])
    on = np.minimum(keep_n, row_half_mirror(send_n))
    ox = np.maximum(keep_x, row_half_mirror(send_x))
    on = np.minimum(on, quad_perm(on, (2, 3, 0, 1)))
    ox = np.maximum(ox, quad_perm(ox, (2, 3, 0, 1)))
    on = np.minimum(on, quad_perm(on, (1, 0, 3, 2)))
    ox = np.maximum(ox, quad_perm(ox, (1, 0, 3, 2)))
    return on, ox


def scatter4_8(mn, mx):
    """minmax_scatter4_8: four rows over groups of 8 lanes."""
    lane = np.arange(LANES)
    b2, b1 = (lane & 4) != 0, (lane & 2) != 0
    kn, kx = [], []
    for i in range(2):
        keep_n, send_n = np.where(b2, mn[2 + i], mn[i]), np.where(b2, mn[i], mn[2 + i])
        keep_x, send_x = np.where(b2, mx[2 + i], mx[i]), np.where(b2, mx[i], mx[2 + i])
        kn.append(np.minimum(keep_n, row_half_mirror(send_n)))
        kx.append(np.maximum(keep_x, row_half_mirror(send_x)))
    keep_n, send_n = np.where(b1, kn[1], kn[0]), np.where(b1, kn[0], kn[1])
    keep_x, send_x = np.where(b1, kx[1], kx[0]), np.where(b1, kx[0], kx[1])
    on = np.minimum(keep_n, quad_perm(send_n, (2, 3, 0, 1)))
    ox = np.maximum(keep_x, quad_perm(send_x, (2, 3, 0, 1)))
    on = np.minimum(on, quad_perm(on, (1, 0, 3, 2)))
    ox = np.maximum(ox, quad_perm(ox, (1, 0, 3, 2)))
    return on, ox


@pytest.mark.parametrize("width", [16, 8])
@pytest.mark.parametrize("seed", range(5))
def test_reduce_scatter_gives_each_lane_one_rows_group_extrema(width, seed):
    rng = np.random.default_rng(seed)
    # distinct values, so that a min or max over the wrong lane set shows
    mn = rng.permutation(4 * LANES).reshape(4, LANES).astype(np.float64)
    mx = rng.permutation(4 * LANES).reshape(4, LANES).astype(np.float64)
    on, ox = (scatter4_16 if width == 16 else scatter4_8)(mn, mx)
    shift = 2 if width == 16 else 1
    for j in range(LANES):
        row = (j >> shift) & 3
        grp = slice(j & ~(width - 1), (j & ~(width - 1)) + width)
        assert on[j] == mn[row, grp].min(), (width, j, row)
        assert ox[j] == mx[row, grp].max(), (width, j, row)


@pytest.mark.parametrize("width", [16, 8])
def test_broadcast_reads_the_rows_lane_in_the_same_group(width):
    """from_quad<P> (16-lane groups: and 0x10, or 4 P) and from_pair<P>
    (8-lane groups: and 0x18, or 2 P) read, for every lane, a lane of its own
    group that holds row P after the reduce-scatter."""
    shift = 2 if width == 16 else 1
    holder_row = (np.arange(LANES) >> shift) & 3
    holder_grp = np.arange(LANES) // width
    for p in range(4):
        if width == 16:
            src_row = swizzle_bitmask(holder_row, 0x10, 4 * p)
            src_grp = swizzle_bitmask(holder_grp, 0x10, 4 * p)
        else:
            src_row = swizzle_bitmask(holder_row, 0x18, 2 * p)
            src_grp = swizzle_bitmask(holder_grp, 0x18, 2 * p)
        assert np.all(src_row == p), (width, p)
        assert np.all(src_grp == holder_grp), (width, p)


def test_swizzle_offsets_match_the_kernels_encoding():
    """The kernels pass (or_mask << 5) | and_mask as the swizzle offset (bit
    15 clear: bitmask mode, xor_mask 0); check that this decodes to the masks
    the broadcast test above uses."""
    for p in range(4):
        for width, and_mask, or_mask in ((16, 0x10, 4 * p), (8, 0x18, 2 * p)):
            off = (or_mask << 5) | and_mask
            assert off & 0x8000 == 0
            assert off & 0x1F == and_mask
            assert (off >> 5) & 0x1F == or_mask
            assert (off >> 10) & 0x1F == 0
