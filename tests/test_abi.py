"""The C-ABI library loads, exports every symbol include/arepi.h declares, and
rejects bad arguments before launching anything (CPU only: no call here
reaches a kernel launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import all_reduce_epilogues_amd as A
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "arepi.h")).read()
    return sorted(set(re.findall(r"\b(arepi_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = A.lib()
    names = declared_symbols()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
        assert getattr(lib, n) is not None


def test_version_and_empty_error():
    assert "gfx950" in A.version()


@pytest.mark.parametrize("M,N,R,ftm,ftn", [
    (256, 512, 2, 128, 128), (4096, 4096, 4, 128, 128), (256, 7168, 8, 128, 128),
    (8192, 7168, 8, 128, 128), (200, 520, 2, 32, 64), (24, 8, 8, 1, 8), (1056, 64, 1, 32, 32),
])
def test_flag_words_agree_with_oracle(M, N, R, ftm, ftn):
    assert A.gemm_rs_flag_words(M, N, R, ftm, ftn) == oracle.flag_words(M, N, R, ftm, ftn)


def nests(M, N, R, ftm, ftn, BM, BN):
    """Brute force: every flag tile lies inside one compute tile."""
    seg = M // R
    for c0 in range(0, N, ftn):
        c1 = min(c0 + ftn, N) - 1
        if c0 // BN != c1 // BN:
            return False
    for d in range(R):
        for r0 in range(0, seg, ftm):
            s, e = d * seg + r0, d * seg + min(r0 + ftm, seg) - 1
            if s // BM != e // BM:
                return False
    return True


TILE_DIMS = A.TILE_DIMS


@pytest.mark.parametrize("M,N,R,ftm,ftn", [
    (256, 512, 2, 128, 128), (256, 7168, 8, 128, 128), (1024, 7168, 8, 128, 128),
    (200, 520, 2, 32, 64), (96, 72, 4, 24, 8), (192, 256, 3, 64, 128), (512, 512, 2, 256, 256),
])
def test_supports_matches_flag_nesting(M, N, R, ftm, ftn):
    for tile, (BM, BN) in TILE_DIMS.items():
        # contiguous row blocks: flag tiles must nest in BM x BN blocks
        rc = A.gemm_rs_supports(M, N, 64, R, 0, ftm, ftn, publish=True, tile=tile)
        assert (rc == 0) == nests(M, N, R, ftm, ftn, BM, BN), (tile, A.last_error())
        # paired half-blocks are a second way to nest them
        rc = A.gemm_rs_supports(M, N, 64, R, 0, ftm, ftn, publish=True, tile=tile | A.TILE_PAIRED_ROWS)
        expect = nests(M, N, R, ftm, ftn, BM, BN) or (paired_eligible(M, R, BM) and
                                                      nests(M, N, R, ftm, ftn, BM // 2, BN))
        assert (rc == 0) == expect, (tile, A.last_error())
        # without publication every tile is allowed
        assert A.gemm_rs_supports(M, N, 64, R, 0, ftm, ftn, publish=False, tile=tile) == 0
        # consuming ready_in bits needs the same nesting as publishing
        rc = A.gemm_rs_supports(M, N, 64, R, 0, ftm, ftn, publish=False, tile=tile | A.TILE_CONSUME_READY)
        assert (rc == 0) == nests(M, N, R, ftm, ftn, BM, BN), (tile, A.last_error())


def paired_eligible(M, R, BM):
    """Half-blocks of BM/2 rows can be paired when every segment is made of whole half-blocks."""
    return R >= 2 and BM >= 64 and (M // R) % (BM // 2) == 0


SCHEDULE_SHAPES = [
    (4096, 4096, 4, 0, 128, 128), (4096, 4096, 4, 2, 128, 128), (8192, 7168, 8, 0, 128, 128),
    (1024, 7168, 8, 5, 128, 128), (256, 7168, 8, 0, 128, 128), (256, 512, 2, 1, 128, 128),
    (384, 520, 3, 1, 64, 64), (640, 264, 5, 4, 64, 8), (200, 520, 2, 1, 32, 64), (640, 384, 1, 0, 128, 128),
    (520, 1032, 8, 4, 128, 128), (1536, 136, 6, 3, 128, 8),
]


@pytest.mark.parametrize("M,N,R,owner,ftm,ftn", SCHEDULE_SHAPES)
def test_schedule_covers_every_output_once(M, N, R, owner, ftm, ftn):
    seg = M // R
    for base, (BM, BN) in TILE_DIMS.items():
        for tile in (base, base | A.TILE_PAIRED_ROWS):
            for publish in (False, True):
                if A.gemm_rs_supports(M, N, 64, R, owner, ftm, ftn, publish=publish, tile=tile) != 0:
                    continue
                sched = A.gemm_rs_schedule(M, N, 64, R, owner, ftm, ftn, publish=publish, tile=tile)
                ncb = -(-N // BN)
                seen = np.zeros((M, ncb), np.int32)
                blocks = set()
                paired = False
                for rb, cb, a0, alen, b0, blen in sched:
                    blocks.add((rb, cb))
                    assert 0 <= cb < ncb
                    for first, n in ((a0, alen), (b0, blen)):
                        assert 0 <= n <= BM
                        if n:
                            seen[first:first + n, cb] += 1
                    if b0 != a0 + alen and blen:
                        paired = True
                assert len(blocks) == len(sched), "a tile is launched twice"
                assert np.all(seen == 1), (tile, publish, "rows covered %s times" % np.unique(seen))
                if paired:
                    CK = BM // 2
                    assert paired_eligible(M, R, BM) and tile & A.TILE_PAIRED_ROWS
                    for rb, cb, a0, alen, b0, blen in sched:
                        for first, n in ((a0, alen), (b0, blen)):
                            # a chunk is a whole half-block inside one segment
                            assert n in (0, CK) and (n == 0 or first // seg == (first + n - 1) // seg)
                        # at most one owner chunk per workgroup: the owner rows are spread out
                        own = sum(1 for first, n in ((a0, alen), (b0, blen)) if n and first // seg == owner)
                        assert own <= 1 or R == 1


def test_auto_tile_is_supported():
    for M in (256, 1024, 4096, 8192):
        t = A.gemm_rs_pick_tile(M, 7168, 2048, 8, 0, 128, 128, publish=True)
        assert A.gemm_rs_supports(M, 7168, 2048, 8, 0, 128, 128, publish=True, tile=t) == 0


@pytest.mark.parametrize("args,needle", [
    ((256, 512, 256, 0, 0), "R=0"),
    ((256, 512, 256, 9, 0), "R=9"),
    ((256, 512, 256, 2, 2), "owner=2"),
    ((255, 512, 256, 2, 0), "not a multiple of R"),
    ((256, 500, 256, 2, 0), "N=500"),
    ((256, 512, 250, 2, 0), "K=250"),
    ((0, 512, 256, 1, 0), "M=0"),
])
def test_gemm_rs_rejects_bad_shapes(args, needle):
    M, N, K, R, owner = args
    rc = A.gemm_rs_supports(M, N, K, R, owner, 128, 128)
    assert rc == A.EINVAL
    assert needle in A.last_error()


def test_gemm_rs_fused_validates_before_launch():
    L = A.lib()
    vp = ctypes.c_void_p
    # NULL x: rejected by name, nothing launched
    rc = L.arepi_gemm_rs_fused(None, None, None, None, None, None, None, 256, 512, 256, 2, 0, 128, 128,
                               0, 0, None, 0, None)
    assert rc == A.EINVAL and "non-NULL" in A.last_error()
    # bad scope value
    buf = ctypes.create_string_buffer(64)
    p = vp(ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16)
    recv = (vp * 2)(None, p)
    rc = L.arepi_gemm_rs_fused(p, p, ctypes.cast(recv, vp), p, p, None, None, 256, 512, 256, 2, 0, 128, 128,
                               7, 0, None, 0, None)
    assert rc == A.EINVAL and "scope=7" in A.last_error()
    # ready_out without send
    rc = L.arepi_gemm_rs_fused(p, p, ctypes.cast(recv, vp), p, p, None, p, 256, 512, 256, 2, 0, 128, 128,
                               0, 0, None, 0, None)
    assert rc == A.EINVAL and "ready_out needs send" in A.last_error()
    # misaligned pointer
    bad = vp(p.value + 2)
    rc = L.arepi_gemm_rs_fused(bad, p, ctypes.cast(recv, vp), p, p, None, None, 256, 512, 256, 2, 0, 128, 128,
                               0, 0, None, 0, None)
    assert rc == A.EINVAL and "aligned" in A.last_error()
    # unknown tile id
    rc = L.arepi_gemm_rs_fused(p, p, ctypes.cast(recv, vp), p, p, None, None, 256, 512, 256, 2, 0, 128, 128,
                               0, 42, None, 0, None)
    assert rc == A.EINVAL and "tile_cfg=42" in A.last_error()
    # flag tiles that straddle the forced compute tile, with publication
    rc = L.arepi_gemm_rs_fused(p, p, ctypes.cast(recv, vp), p, p, p, p, 256, 512, 256, 2, 0, 128, 128,
                               0, A.TILE_64x128, None, 0, None)
    assert rc == A.EUNSUPPORTED and "straddle" in A.last_error()


def test_lamport_and_combine_validate_before_launch():
    L = A.lib()
    assert L.arepi_ar_rmsnorm_lamport(None, None, None, 4, 64, 9, 1e-6, 0, None, 0, None) == A.EINVAL
    assert "S=9" in A.last_error()
    assert L.arepi_ar_rmsnorm_lamport(None, None, None, 4, 20000, 8, 1e-6, 0, None, 0, None) == A.EUNSUPPORTED
    assert L.arepi_ar_rmsnorm_lamport(None, None, None, 4, 60, 8, 1e-6, 0, None, 0, None) == A.EINVAL
    assert L.arepi_ar_rmsnorm_lamport(None, None, None, 4, 64, 8, 1e-6, 0, None, 0, None) == A.EINVAL
    assert "non-NULL" in A.last_error()
    assert L.arepi_ar_rmsnorm_lamport(None, None, None, 0, 64, 8, 1e-6, 0, None, 0, None) == A.OK  # empty
    assert L.arepi_lamport_publish(None, None, None, 8, 4, 64, 128, 12, 0, None) == A.EINVAL
    assert L.arepi_lamport_prefill(None, -1, None) == A.EINVAL
    assert L.arepi_lamport_prefill(None, 0, None) == A.OK
    assert L.arepi_combine_reduce(None, None, None, 4, 17, 64, None) == A.EUNSUPPORTED
    assert "E=17" in A.last_error()
    assert L.arepi_combine_reduce_lds(None, None, None, 4, 17, 64, None) == A.EUNSUPPORTED
    assert L.arepi_combine_reduce_lds(None, None, None, 4, 8, 64, None) == A.EINVAL
    assert L.arepi_combine_reduce(None, None, None, 4, 8, 60, None) == A.EINVAL
    assert L.arepi_combine_reduce(None, None, None, 0, 8, 64, None) == A.OK  # empty: nothing to do
    assert L.arepi_combine_reduce(None, None, None, 4, 8, 64, None) == A.EINVAL
    assert L.arepi_emu_peer_producer(None, None, None, None, 1, 256, 512, 2, 5, 128, 128, 0, 0, 1, None, None) == A.EINVAL
    assert L.arepi_emu_peer_producer(None, None, None, None, 1, 256, 512, 2, 0, 128, 128, 0, 0, 0, None, None) == A.EINVAL
    assert "items_per_release" in A.last_error()
    assert L.arepi_emu_producer_gate(None, None, 0, None) == A.EINVAL
    assert "resident" in A.last_error()
    assert L.arepi_emu_peer_producer_steps(None, None, None, None, 1, 1, 256, 512, 2, 0, 128, 128, 0, 0, 1,
                                           None, None, 0, 2, 0, None, 0, None) == A.EINVAL
    assert "go" in A.last_error()
    go = ctypes.c_void_p(16)  # never dereferenced: the calls below fail validation first
    assert L.arepi_emu_peer_producer_steps(None, None, None, None, 1, 1, 256, 512, 2, 0, 128, 128, 0, 0, 1,
                                           None, go, 2, 2, 0, None, 0, None) == A.EINVAL
    assert "credit" in A.last_error()
    assert L.arepi_emu_peer_producer_steps(None, None, None, None, 1, 1, 256, 512, 2, 0, 128, 128, 0, 0, 1,
                                           None, go, 1, 2, 12, None, 0, None) == A.EINVAL
    assert "src_step" in A.last_error()
    assert L.arepi_emu_peer_producer_steps(None, None, None, None, 1, 1, 256, 512, 2, 0, 128, 128, 0, 0, 1,
                                           None, go, 1, 0, 0, None, 0, None) == A.EINVAL
    assert "steps" in A.last_error()
    assert L.arepi_emu_peer_producer_steps(None, None, None, None, 1, 1, 256, 512, 2, 0, 128, 128, 0, 0, 1,
                                           None, go, 1, 2, 0, None, 0, None) == A.EINVAL
    assert "non-NULL" in A.last_error()
    assert L.arepi_emu_signal(None, 1, None) == A.EINVAL


def test_noalloc_consumer_refuses_sizes_beyond_its_static_staging():
    """The limit is checked before any device call: the row just past it is
    refused as unsupported, the largest row count that fits passes the size
    check and then fails on the NULL pointers."""
    L = A.lib()
    S, N = 8, 7168
    rows = A.LAMPORT_NOALLOC_BYTES // (S * N * 2)
    assert rows == 292
    rc = L.arepi_ar_rmsnorm_lamport_noalloc(None, None, rows + 1, N, S, 1e-6, 0, None, 0, None, None)
    assert rc == A.EUNSUPPORTED and "static staging" in A.last_error()
    rc = L.arepi_ar_rmsnorm_lamport_noalloc(None, None, rows, N, S, 1e-6, 0, None, 0, None, None)
    assert rc == A.EINVAL and "non-NULL" in A.last_error()
    rc = L.arepi_ar_rmsnorm_lamport_noalloc(None, None, 4, 64, 9, 1e-6, 0, None, 0, None, None)
    assert rc == A.EINVAL and "S=9" in A.last_error()
    rc = L.arepi_ar_rmsnorm_lamport_noalloc(None, None, 1 << 40, 16384, 8, 1e-6, 0, None, 0, None, None)
    assert rc == A.EUNSUPPORTED  # no overflow in the size check


def test_binding_checks_dtype_before_pointers():
    import torch
    x = torch.zeros(4, 8, dtype=torch.float32)
    with pytest.raises(TypeError):
        A.combine_reduce(x, x, x)


@pytest.mark.parametrize("M,N,R", [(4096, 4096, 4), (8192, 7168, 8), (4096, 7168, 8)])
def test_owner_half_blocks_pair_on_the_model_shapes(M, N, R):
    seg = M // R
    tile = A.gemm_rs_pick_tile(M, N, 2048, R, 0, publish=True)
    BM = A.TILE_DIMS[tile][0]
    sched = A.gemm_rs_schedule(M, N, 2048, R, 0, publish=True, tile=tile | A.TILE_PAIRED_ROWS)
    owner_wgs = [s for s in sched if s[2] // seg == 0 or (s[5] and s[4] // seg == 0)]
    # every workgroup holding owner rows holds exactly one half-block of them, next to a non-owner one
    assert len(owner_wgs) == (seg // (BM // 2)) * (-(-N // A.TILE_DIMS[tile][1]))
    for rb, cb, a0, alen, b0, blen in owner_wgs:
        assert a0 // seg == 0 and alen == BM // 2 and blen == BM // 2 and b0 // seg != 0


@pytest.mark.parametrize("M,N,R", [(4096, 4096, 4), (1024, 7168, 8), (200, 520, 2)])
def test_consume_option_plans_like_publication(M, N, R):
    """AREPI_TILE_CONSUME_READY picks and lays out tiles as publication does
    (both need every flag tile under one workgroup).  The automatic owner
    half-height tiles are the one difference: consumed bits also need each
    flag tile under one owner tile, published ones do not."""
    for ftm, ftn in ((128, 128), (32, 64)):
        auto = A.gemm_rs_pick_tile(M, N, 2048, R, 0, ftm, ftn, publish=True)
        if auto < 0:
            assert A.gemm_rs_supports(M, N, 2048, R, 0, ftm, ftn, tile=A.TILE_CONSUME_READY) < 0
            continue
        ref = A.gemm_rs_schedule(M, N, 2048, R, 0, ftm, ftn, publish=True, tile=auto)
        got = A.gemm_rs_schedule(M, N, 2048, R, 0, ftm, ftn, publish=False, tile=auto | A.TILE_CONSUME_READY)
        assert np.array_equal(ref, got)
        half_pub = any(w[0] == -1 for w in A.gemm_rs_schedule(M, N, 2048, R, 0, ftm, ftn, publish=True))
        half_con = any(w[0] == -1 for w in A.gemm_rs_schedule(M, N, 2048, R, 0, ftm, ftn, publish=False,
                                                                tile=A.TILE_CONSUME_READY))
        owner_rows = A.TILE_DIMS[auto][0] // 2
        assert half_con == (half_pub and owner_rows % ftm == 0)


@pytest.mark.parametrize("M,N,R,owner", [(4096, 7168, 8, 3), (8192, 7168, 8, 0), (1024, 7168, 8, 5),
                                         (4096, 4096, 4, 0), (520, 1032, 8, 4), (200, 520, 2, 1)])
def test_owner_first_reorders_the_same_tiles(M, N, R, owner):
    """AREPI_TILE_OWNER_FIRST keeps the tile set and layout and moves the
    workgroups holding owner rows ahead of the rest; where the default order
    leaves them for a second round of 256 workgroups, the owner-first order
    puts them all in the first."""
    seg = M // R
    pub = A.gemm_rs_supports(M, N, 2048, R, owner, publish=True) == 0
    # the explicit tile of the automatic choice (AUTO alone may also split the
    # owner rows into half-height tiles, which the owner-first order does not)
    tile = A.gemm_rs_pick_tile(M, N, 2048, R, owner, publish=pub)
    base = np.asarray(A.gemm_rs_schedule(M, N, 2048, R, owner, publish=pub, tile=tile))
    first = np.asarray(A.gemm_rs_schedule(M, N, 2048, R, owner, publish=pub, tile=tile | A.TILE_OWNER_FIRST))
    assert sorted(map(tuple, base.tolist())) == sorted(map(tuple, first.tolist()))

    def owner_rows(s):
        return np.array([a0 // seg == owner or (blen > 0 and b0 // seg == owner) for _, _, a0, _, b0, blen in s])
    ob, of = owner_rows(base), owner_rows(first)
    idx = np.arange(len(base))
    if ob.all():
        return  # one segment holds every tile: nothing to reorder
    assert idx[of].mean() < idx[~of].mean() and idx[ob].mean() > idx[~ob].mean()
    if len(base) > 256 and of.sum() <= 256:
        assert idx[of].max() < 256 and idx[ob].min() >= len(base) - 256 - 32


@pytest.mark.parametrize("M,N,R,owner,tile", [(4096, 7168, 8, 0, 0), (4096, 7168, 8, 3, 11), (8192, 7168, 8, 5, 0),
                                              (2048, 4096, 4, 1, 11), (512, 520, 2, 1, 11), (2048, 1032, 8, 7, 11),
                                              (1024, 7168, 8, 3, 0), (1024, 1032, 8, 0, 2), (384, 520, 3, 2, 2)])
def test_owner_half_tiles_cover_the_owner_segment_last(M, N, R, owner, tile):
    """AREPI_TILE_OWNER_HALF: the owner segment's rows leave the BM x 256
    schedule and come after it as BM/2 x 256 workgroups (two BM/4-row chunks,
    row block -1), one per half-block and column block; every row and column
    block is covered exactly once, and no workgroup before them holds owner
    rows."""
    seg = M // R
    BM = A.TILE_DIMS[tile or A.gemm_rs_pick_tile(M, N, 2048, R, owner, publish=True)][0]
    sched = np.asarray(A.gemm_rs_schedule(M, N, 2048, R, owner, publish=True, tile=tile | A.TILE_OWNER_HALF))
    ncb = -(-N // 256)
    n_half = 2 * (seg // BM) * ncb
    assert len(sched) == (M // BM) * ncb - (seg // BM) * ncb + n_half
    head, tail = sched[:-n_half], sched[-n_half:]
    assert not any(a0 // seg == owner or (blen and b0 // seg == owner) for _, _, a0, _, b0, blen in head)
    assert (tail[:, 0] == -1).all() and (tail[:, 3] == BM // 4).all() and (tail[:, 5] == BM // 4).all()
    assert (tail[:, 4] == tail[:, 2] + BM // 4).all() and ((tail[:, 2] - owner * seg) % (BM // 2) == 0).all()
    cover = np.zeros((M, ncb), np.int32)
    for rb, cb, a0, alen, b0, blen in sched:
        cover[a0:a0 + alen, cb] += 1
        cover[b0:b0 + blen, cb] += 1
    assert (cover == 1).all()


def test_automatic_choice_uses_owner_half_tiles_where_no_round_is_added():
    """AUTO splits the owner rows into half-height tiles when that keeps the
    number of 256-workgroup rounds (tp=8 M = 1024, 2048, 4096, 8192), not for
    the one-round tp=4 share (256 -> 320 workgroups), not where consumed flag
    tiles would straddle two owner tiles, and never when an explicit tile is
    given."""
    def half(M, N, R, tile=A.TILE_AUTO, ftm=128, publish=True):
        s = A.gemm_rs_schedule(M, N, 2048, R, 0, ftm, 128, publish=publish, tile=tile)
        return any(w[0] == -1 for w in s), len(s)
    assert half(4096, 4096, 4) == (False, 256)
    assert half(2048, 7168, 8) == (True, 252)
    assert half(4096, 7168, 8) == (True, 504)
    assert half(8192, 7168, 8) == (True, 1008)
    assert half(1024, 7168, 8) == (True, 252)  # 128x256 tiles, owner rows as 64x256: still one round
    assert half(4096, 7168, 8, tile=A.TILE_256x256_W8_K64) == (False, 448)
    assert half(4096, 7168, 8, tile=A.TILE_CONSUME_READY, ftm=256, publish=False)[0] is False
    assert half(4096, 7168, 8, tile=A.TILE_CONSUME_READY, ftm=128, publish=False)[0] is True
    assert half(1024, 7168, 8, tile=A.TILE_CONSUME_READY, ftm=128, publish=False)[0] is False  # 64-row owner tiles


def test_owner_half_refusals():
    t = A.TILE_OWNER_HALF
    assert A.gemm_rs_supports(4096, 7168, 2048, 8, 0, publish=True, tile=t) == 0
    assert A.gemm_rs_supports(4096, 7168, 2048, 8, 0, publish=True, tile=t | A.TILE_256x256_W8_K64) == 0
    assert A.gemm_rs_supports(4096, 7168, 2048, 8, 0, publish=True, tile=t | A.TILE_256x256_W8_K64
                              | A.TILE_PAIRED_ROWS) == A.EINVAL
    assert A.gemm_rs_supports(4096, 7168, 2048, 8, 0, publish=True, tile=t | A.TILE_OWNER_FIRST) == A.EINVAL
    assert A.gemm_rs_supports(4096, 7168, 2048, 8, 0, publish=True, tile=t | A.TILE_128x256) == 0
    assert A.gemm_rs_supports(4096, 7168, 2048, 8, 0, publish=True, tile=t | A.TILE_128x128) == A.EUNSUPPORTED
    assert "AREPI_TILE_128x256" in A.last_error()
    assert A.gemm_rs_supports(1024, 7168, 2048, 8, 0, publish=True, tile=t | A.TILE_256x256_W8_K64) == \
        A.EUNSUPPORTED  # 128-row segments
    assert A.gemm_rs_supports(1024, 7168, 2048, 8, 0, publish=True, tile=t) == 0  # AUTO picks 128x256
    assert A.gemm_rs_supports(4096, 7168, 2048, 1, 0, publish=True, tile=t | A.TILE_256x256_W8_K64) == \
        A.EUNSUPPORTED
    # 256-row flag tiles straddle the 128-row owner tiles: fine for waiting, not for consuming
    assert A.gemm_rs_supports(4096, 7168, 2048, 8, 0, 256, 256, publish=True, tile=t | A.TILE_256x256_W8_K64) == 0
    assert A.gemm_rs_supports(4096, 7168, 2048, 8, 0, 256, 256, publish=True,
                              tile=t | A.TILE_256x256_W8_K64 | A.TILE_CONSUME_READY) == A.EUNSUPPORTED
    assert A.gemm_rs_ring_supports(4096, 7168, 2048, 8, 0, publish=True, tile=t) == A.EINVAL
    assert A.gemm_rs_fp8_supports(512, 512, 256, 2, 0, tile=t) != 0


def test_owner_first_refuses_paired_rows_ring_and_fp8():
    t = A.TILE_OWNER_FIRST
    assert A.gemm_rs_supports(4096, 4096, 2048, 4, 0, publish=True, tile=t) == 0
    assert A.gemm_rs_supports(4096, 4096, 2048, 4, 0, publish=True, tile=t | A.TILE_PAIRED_ROWS) == A.EINVAL
    assert "contiguous" in A.last_error()
    assert A.gemm_rs_ring_supports(4096, 4096, 2048, 4, 0, publish=True, tile=t) == A.EINVAL
    assert "ring" in A.last_error()
    assert A.gemm_rs_fp8_supports(512, 512, 256, 2, 0, tile=t) != 0


@pytest.mark.parametrize("M,N,R,owner", [(256, 512, 2, 0), (4096, 4096, 4, 0), (256, 7168, 8, 0), (96, 72, 4, 2)])
def test_ring_supports_follows_the_direct_form(M, N, R, owner):
    """The push-ring form accepts what the direct form accepts (contiguous
    rows), refuses paired half-blocks, and needs 8-row-aligned segments; when
    it publishes, every row block must also lie in one segment (tile rows
    dividing M/R), and the automatic choice keeps to such tiles."""
    seg = M // R
    whole = [t for t in TILE_DIMS if seg % TILE_DIMS[t][0] == 0 and
             A.gemm_rs_supports(M, N, 64, R, owner, 128, 128, publish=True, tile=t) == 0]
    for tile in TILE_DIMS:
        for publish in (False, True):
            d = A.gemm_rs_supports(M, N, 64, R, owner, 128, 128, publish=publish, tile=tile)
            r = A.gemm_rs_ring_supports(M, N, 64, R, owner, 128, 128, publish=publish, tile=tile)
            if publish and R > 1 and d == 0 and seg % TILE_DIMS[tile][0]:
                assert r == A.EUNSUPPORTED and "segment height" in A.last_error(), (tile, A.last_error())
            else:
                assert r == d, (tile, publish, A.last_error())
    auto = A.gemm_rs_ring_supports(M, N, 64, R, owner, 128, 128, publish=True)
    if R > 1 and seg % 8 == 0:
        assert (auto == 0) == bool(whole), A.last_error()
    if auto == 0 and R > 1:
        assert A.gemm_rs_ring_pick_tile(M, N, 64, R, owner, publish=True) in whole
        assert A.gemm_rs_ring_supports(M, N, 64, R, owner, 128, 128, tile=tile | A.TILE_PAIRED_ROWS) == \
            A.EUNSUPPORTED
        assert "direct form only" in A.last_error()


def test_ring_rejects_unaligned_segments_and_bad_pointers():
    assert A.gemm_rs_ring_supports(24, 8, 16, 8, 7, 3, 8) == A.EUNSUPPORTED
    assert "multiple of 8" in A.last_error()
    assert A.gemm_rs_ring_supports(24, 8, 16, 1, 0, 3, 8) == 0  # one rank: no segments to align
    L = A.lib()
    vp = ctypes.c_void_p
    buf = ctypes.create_string_buffer(64)
    p = vp(ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16)
    # R=4, owner=1: chain segment 0 may be NULL, segment 3 may not
    up = (vp * 4)(None, p, p, None)
    rc = L.arepi_gemm_rs_ring(p, p, ctypes.cast(up, vp), p, p, p, None, 256, 512, 256, 4, 1, 128, 128,
                              0, 0, None, 0, None)
    assert rc == A.EINVAL and "upstream[3]" in A.last_error()
    up = (vp * 4)(None, p, p, p)
    rc = L.arepi_gemm_rs_ring(p, p, ctypes.cast(up, vp), p, p, None, None, 256, 512, 256, 4, 1, 128, 128,
                              0, 0, None, 0, None)
    assert rc == A.EINVAL and "send" in A.last_error()
    rc = L.arepi_gemm_rs_ring(p, p, ctypes.cast(up, vp), None, p, p, None, 256, 512, 256, 4, 1, 128, 128,
                              0, 0, None, 0, None)
    assert rc == A.EINVAL and "ready_in" in A.last_error()
    rc = L.arepi_gemm_rs_ring(p, p, ctypes.cast(up, vp), p, p, p, None, 256, 512, 256, 4, 1, 128, 128,
                              3, 0, None, 0, None)
    assert rc == A.EINVAL and "scope=3" in A.last_error()


@pytest.mark.parametrize("M,N,R,ftm,ftn", [
    (256, 512, 2, 128, 128), (1024, 7168, 8, 128, 128), (4096, 4096, 4, 128, 128),
    (200, 520, 2, 32, 64), (512, 512, 2, 256, 256), (512, 384, 2, 128, 128), (1024, 1024, 4, 64, 256),
])
def test_fp8_supports_nests_flag_tiles_in_its_256x256_tile(M, N, R, ftm, ftn):
    K = 256
    rc = A.gemm_rs_fp8_supports(M, N, K, R, 0, ftm, ftn, publish=True)
    assert (rc == 0) == nests(M, N, R, ftm, ftn, 256, 256), A.last_error()
    rc = A.gemm_rs_fp8_supports(M, N, K, R, 0, ftm, ftn, publish=False, tile=A.TILE_CONSUME_READY)
    assert (rc == 0) == nests(M, N, R, ftm, ftn, 256, 256), A.last_error()
    assert A.gemm_rs_fp8_supports(M, N, K, R, 0, ftm, ftn, publish=False) == 0


def test_fp8_supports_rejects_k_and_tile_options():
    assert A.gemm_rs_fp8_supports(512, 512, 192, 2, 0) != 0
    assert "multiple of 128" in A.last_error()
    assert A.gemm_rs_fp8_supports(512, 512, 256, 2, 0, tile=A.TILE_256x256_W8_K64) != 0
    assert A.gemm_rs_fp8_supports(512, 512, 256, 2, 0, tile=A.TILE_PAIRED_ROWS) != 0
    assert A.gemm_rs_fp8_supports(512, 512, 256, 2, 0, tile=A.TILE_CONSUME_READY) == 0
