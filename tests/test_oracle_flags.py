"""Pins for the per-tile readiness bitmask geometry (CPU only).

The expected words are rebuilt here by walking every element of every segment
and marking the flag tile it falls in -- a different formulation from the
oracle's ceil-division count.
"""
import numpy as np
import pytest

import oracle


def brute_force_words(M, N, R, owner, ftm, ftn):
    seg = M // R
    # tile id of each (row, col) of a segment, numbered row-major by first appearance
    ids = {}
    for r in range(seg):
        for c in range(N):
            key = (r // ftm, c // ftn)
            if key not in ids:
                ids[key] = None
    keys = sorted(ids)
    tiles = len(keys)
    W = (tiles + 31) // 32
    words = np.zeros((R, W), dtype=np.uint32)
    for d in range(R):
        if d == owner:
            continue
        for t in range(tiles):
            words[d, t // 32] |= np.uint32(1 << (t % 32))
    return tiles, words


@pytest.mark.parametrize("M,N,R,owner,ftm,ftn", [
    (256, 512, 2, 0, 128, 128),     # tiny workload: 4 tiles per segment
    (256, 512, 2, 1, 128, 128),
    (64, 200, 4, 3, 16, 64),        # ragged right edge
    (96, 96, 2, 0, 40, 40),         # ragged bottom and right edges
    (256, 384, 8, 0, 128, 128),     # 32-row segments clip 128-row tiles
    (40, 8, 8, 5, 128, 128),        # one tile per segment
    (1024, 1024, 2, 1, 32, 32),     # 512 tiles per segment: 16 full words
    (64, 1056, 2, 0, 32, 32),       # 33 tiles: second word has one bit
])
def test_ready_out_matches_brute_force(M, N, R, owner, ftm, ftn):
    tiles, words = brute_force_words(M, N, R, owner, ftm, ftn)
    assert oracle.flag_tiles(M, N, R, ftm, ftn) == tiles
    assert oracle.flag_words(M, N, R, ftm, ftn) == words.shape[1]
    assert np.array_equal(oracle.ready_out(M, N, R, owner, ftm, ftn), words)


def test_flag_geometry_rejects_bad_shapes():
    assert oracle.flag_tiles(10, 8, 4, 8, 8) == -1   # 10 rows do not split 4 ways
    assert oracle.flag_tiles(8, 8, 2, 0, 8) == -1
