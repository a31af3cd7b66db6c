"""Forward progress of the cross-tile carries, checked on the host (no GPU).

A tile that needs a carry waits for tiles farther along the scan direction,
never the other way round.  Those waits end only if every tile a block waits
for belongs to a block of LOWER index: a dispatch starts its workgroups in
index order, so such a block has started, and a started block publishes its
aggregate before it waits for anything.  lrs_debug_schedule runs the
library's own planning and tile-placement code (the functions the kernels
call) and returns the block -> tile map of a call; this file derives from the
shape alone which tiles each tile may wait for and checks the ordering for
every schedule the host can pick: flat and position-major order, every forced
tile shape, forced time-major wave counts, both scan directions, fp32, fp64
and 16-bit plans.

Which tiles a tile may wait for (row-major, tiles of K elements over rows of
T): a tile whose far-boundary element (its last element for a backward scan,
its first for a forward one) is not a row end takes a carry from the adjacent
far tile; that tile's aggregate ends the look-back if it holds a row end,
otherwise the look-back goes on to the next one.  So checking, for every tile
with an open far boundary, that the adjacent far tile's block comes first,
covers every wait by induction along the row.  Time-major: every tile but the
far-most along time waits for the next one farther along time (same
environment group).
"""
import ctypes

import numpy as np
import pytest

from linear_recurrence_scan_env_amd import api, build


class Info(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("num_tiles", ctypes.c_int64),
                ("tile_elems", ctypes.c_int64), ("tile_steps", ctypes.c_int64),
                ("groups", ctypes.c_int64), ("envs_per_group", ctypes.c_int64),
                ("time_major", ctypes.c_int32), ("carries", ctypes.c_int32),
                ("backward", ctypes.c_int32), ("tiles_per_row", ctypes.c_int32),
                ("elems_per_lane", ctypes.c_int32), ("waves_per_block", ctypes.c_int32),
                ("composition_fp64", ctypes.c_int32), ("reserved", ctypes.c_int32)]


TRUNC, REVERSE, TIME_MAJOR, HALF = 1, 2, 4, 8
GAE, VTRACE, RETRACE, LAMBDA, DISC, ELIG, PREFIX_I32, PREFIX_F32, AFFINE = range(9)
BACKWARD_EST = (GAE, VTRACE, RETRACE, LAMBDA, DISC)
TILES = [(4, 1), (4, 4), (8, 4), (4, 8), (16, 4), (4, 16), (8, 16)]


@pytest.fixture(scope="module")
def lib():
    if build.stale():
        build.build()
    lib = api.load()
    lib.lrs_debug_schedule.restype = ctypes.c_int
    lib.lrs_debug_schedule.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_float, ctypes.POINTER(Info),
                                       ctypes.c_void_p, ctypes.c_int64]
    yield lib
    lib.lrs_debug_set_schedule(0, 0, 0)
    lib.lrs_debug_set_time_major_waves(0)


def schedule(lib, est, flags, n, t, beta_max):
    info = Info()
    assert lib.lrs_debug_schedule(est, flags, n, t, beta_max, ctypes.byref(info), None, 0) == 0, \
        lib.lrs_last_error()
    tiles = np.empty(info.num_blocks, dtype=np.uint32)
    assert lib.lrs_debug_schedule(est, flags, n, t, beta_max, ctypes.byref(info),
                                  tiles.ctypes.data, tiles.size) == 0
    return info, tiles.astype(np.int64)


def owners(tiles, num_tiles):
    """owner[tile] = block; the map must be a permutation of the tiles."""
    assert tiles.size == num_tiles
    owner = np.full(num_tiles, -1, dtype=np.int64)
    owner[tiles] = np.arange(tiles.size)
    assert (owner >= 0).all(), "some tile has no block"
    return owner


def row_major_violations(n, t, tile_elems, backward, owner):
    """Tiles whose adjacent far tile (which they may wait for) is owned by a
    block of equal or higher index."""
    total = n * t
    num_tiles = owner.size
    i = np.arange(num_tiles, dtype=np.int64)
    if backward:
        far_elem = np.minimum((i + 1) * tile_elems, total) - 1
        open_ = (far_elem % t) != t - 1
        j = i + 1
    else:
        far_elem = i * tile_elems
        open_ = (far_elem % t) != 0
        j = i - 1
    waits = open_ & (j >= 0) & (j < num_tiles)
    bad = waits & (owner[np.clip(j, 0, num_tiles - 1)] >= owner[i])
    return int(waits.sum()), np.flatnonzero(bad)


def time_major_violations(info, owner):
    tt = info.num_tiles // info.groups
    k = np.arange(tt)[:, None]
    g = np.arange(info.groups)[None, :]
    me = owner[(k * info.groups + g)]
    far = k + (1 if info.backward else -1)
    waits = (far >= 0) & (far < tt) & np.ones_like(g, dtype=bool)
    other = owner[np.clip(far, 0, tt - 1) * info.groups + g]
    return int(waits.sum()), np.argwhere(waits & (other >= me))


def check_call(lib, est, flags, n, t, beta_max):
    info, tiles = schedule(lib, est, flags, n, t, beta_max)
    owner = owners(tiles, info.num_tiles)
    if info.time_major:
        assert info.num_blocks == info.num_tiles
        waits, bad = time_major_violations(info, owner) if info.carries else (0, [])
    else:
        assert info.num_tiles * info.tile_elems >= n * t > (info.num_tiles - 1) * info.tile_elems
        waits, bad = (row_major_violations(n, t, info.tile_elems, bool(info.backward), owner)
                      if info.carries else (0, []))
    assert len(bad) == 0, (est, flags, n, t, info.tile_elems, info.tiles_per_row, bad[:5])
    return info, waits


SHAPES = [(1, 1), (3, 5), (1, 4097), (5, 3001), (64, 131072), (1024, 16384), (1100, 4096),
          (2048, 8192), (4096, 128), (4096, 2048), (33, 2049), (7, 7000003), (3, 100000)]
CALLS = [(e, f) for e in BACKWARD_EST for f in (0, TRUNC)] + \
        [(ELIG, 0), (PREFIX_F32, 0), (PREFIX_I32, 0)] + \
        [(AFFINE, f) for f in (0, TRUNC, REVERSE, TRUNC | REVERSE)]


@pytest.mark.parametrize("half", [0, HALF])
@pytest.mark.parametrize("beta_max", [0.9, 1.0])
def test_row_major_automatic_schedules(lib, half, beta_max):
    lib.lrs_debug_set_schedule(0, 0, 0)
    seen = set()
    for est, flags in CALLS:
        if half and est == PREFIX_I32:
            continue
        for n, t in SHAPES:
            info, waits = check_call(lib, est, flags | half, n, t, beta_max)
            seen.add((info.carries, info.tiles_per_row > 1, bool(info.backward)))
    # both look-back orders, both directions, and whole-row launches were covered
    assert {(1, False, True), (1, False, False), (1, True, True), (1, True, False),
            (0, False, True)} <= seen


@pytest.mark.parametrize("tile", TILES, ids=lambda x: f"{x[0]}x{x[1]}")
def test_row_major_forced_tiles(lib, tile):
    try:
        assert lib.lrs_debug_set_schedule(1, *tile) == 0
        total_waits = 0
        for est, flags in CALLS:
            for n, t in [(1, 4097), (5, 3001), (64, 131072), (2048, 8192), (1024, 4096), (3, 77)]:
                info, waits = check_call(lib, est, flags, n, t, 0.95)
                assert info.carries and (info.elems_per_lane, info.waves_per_block) == tile
                total_waits += waits
        assert total_waits > 0
    finally:
        lib.lrs_debug_set_schedule(0, 0, 0)


@pytest.mark.parametrize("waves", [0, 2, 4, 8, 16])
def test_time_major_schedules(lib, waves):
    try:
        assert lib.lrs_debug_set_time_major_waves(waves) == 0
        any_carry = False
        for est, flags in CALLS:
            for n, t in [(1, 1), (64, 131072), (4096, 128), (4096, 2048), (100, 1000), (4099, 33),
                         (7, 300000), (8200, 1030)]:
                info, waits = check_call(lib, est, flags | TIME_MAJOR, n, t, 0.95)
                any_carry = any_carry or bool(info.carries and waits)
        assert any_carry
    finally:
        lib.lrs_debug_set_time_major_waves(0)


def test_schedule_info_matches_plan(lib):
    """Spot checks of the plans the tuning notes describe."""
    info, _ = schedule(lib, RETRACE, TRUNC, 4096, 128, 0.9405)
    assert (info.carries, info.tile_elems) == (0, 256)          # whole rows, 4 x 1 tiles
    # look-back on 4096-element tiles, or 2048 when fewer than 128 of those
    info, _ = schedule(lib, RETRACE, 0, 4096, 100, 0.9405)       # 100 tiles of 4096
    assert (info.carries, info.tile_elems) == (1, 2048)
    info, _ = schedule(lib, AFFINE, 0, 2048, 300, float("inf"))  # 150 tiles of 4096
    assert (info.carries, info.tile_elems) == (1, 4096)
    info, _ = schedule(lib, GAE, TRUNC, 64, 131072, 0.9405)
    assert (info.carries, info.tile_elems, info.tiles_per_row) == (1, 2048, 0)  # flat look-back
    info, _ = schedule(lib, GAE, 0, 2048, 8192, 0.9405)
    assert (info.carries, info.tile_elems) == (0, 8192)         # whole rows, 8 x 16 tiles
    info, _ = schedule(lib, GAE, 0, 1024, 16384, 0.9405)
    assert info.carries == 1 and info.tiles_per_row == 16384 // info.tile_elems  # position-major
    info, _ = schedule(lib, PREFIX_F32, 0, 64, 131072, 1.0)
    assert info.composition_fp64 == 1 and info.elems_per_lane == 8 and info.waves_per_block == 16
    info, _ = schedule(lib, GAE, 0, 64, 131072, 0.9405)
    assert info.composition_fp64 == 0
    info, _ = schedule(lib, GAE, TIME_MAJOR, 4096, 128, 0.9)
    assert (info.carries, info.envs_per_group, info.groups) == (0, 32, 128)
    info, _ = schedule(lib, GAE, TIME_MAJOR, 64, 131072, 0.9)
    assert (info.carries, info.tile_steps, info.groups) == (1, 256, 1)
    # many environments: two groups of 64 per block, 128-step tiles
    info, _ = schedule(lib, GAE, TIME_MAJOR, 4096, 2048, 0.9)
    assert (info.envs_per_group, info.tile_steps, info.groups, info.waves_per_block) == (128, 128, 32, 16)
    info, _ = schedule(lib, GAE, TIME_MAJOR, 8192, 512, 0.9)
    assert (info.envs_per_group, info.tile_steps) == (128, 128)
    for n, t in [(4096, 512), (2048, 8192), (4096, 256)]:
        info, _ = schedule(lib, DISC, TIME_MAJOR, n, t, 0.9)
        assert (info.envs_per_group, info.tile_steps) == (64, 256), (n, t)
    # one block per CU and 256-step tiles would leave CUs idle: 128-step tiles
    # (fewer than 256 blocks of 256 steps), for the calls the capped kernel
    # cannot take, including discounted returns with maps composed in fp64
    for est, bm in [(GAE, 0.9), (VTRACE, 0.9), (RETRACE, 0.9), (DISC, 0.995)]:
        info, _ = schedule(lib, est, TIME_MAJOR, 4096, 512, bm)
        assert (info.tile_steps, info.elems_per_lane, info.groups) == (128, 8, 64), est
    info, _ = schedule(lib, GAE, TIME_MAJOR, 4096, 769, 0.9)  # 64 x 4 blocks: enough
    assert info.tile_steps == 256
    info, _ = schedule(lib, GAE, TIME_MAJOR, 4096, 768, 0.9)  # 64 x 3 blocks: few
    assert info.tile_steps == 128
    assert lib.lrs_debug_schedule(99, 0, 4, 4, 0.5, ctypes.byref(info), None, 0) == 1
    assert lib.lrs_debug_schedule(GAE, REVERSE, 4, 4, 0.5, ctypes.byref(info), None, 0) == 1
    assert lib.lrs_debug_schedule(PREFIX_I32, HALF, 4, 4, 0.5, ctypes.byref(info), None, 0) == 1
    assert lib.lrs_debug_schedule(GAE, 0, 0, 4, 0.5, ctypes.byref(info), None, 0) == 1


def test_checker_rejects_a_paired_tile_mapping():
    """Negative control: a mapping in which block b works on two tiles at
    distance D (i and i + D of each group of 2D tiles) makes the first block
    of a group wait for the group's last block (tile D, forward, needs tile
    D - 1 of block D - 1), which violates the ordering: such a launch completes
    only while all D blocks of a group are resident at once.  A mapping of
    this kind was tried as a variant and dropped; the check above would have
    flagged it."""
    n, t, k, d = 1, 4 * 512 * 256, 256, 512  # one row of 2048 tiles of 4 x 1
    num_tiles = n * t // k
    owner = np.empty(num_tiles, dtype=np.int64)
    for b in range(num_tiles // 2):
        grp, i = divmod(b, d)
        owner[2 * grp * d + i] = b
        owner[2 * grp * d + d + i] = b
    # two tiles per block: a tile may also "wait" on a tile of its own block;
    # only strictly lower blocks are safe, so count both as violations
    _, bad = row_major_violations(n, t, k, False, owner)
    assert len(bad) > 0
    assert 512 in bad  # tile D (block 0's second tile) waits for tile D-1 of block D-1
