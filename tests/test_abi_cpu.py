"""The C-ABI library without a GPU: it loads, exports every symbol its header
declares, and rejects bad arguments on the host before any HIP call."""

import os
import re

import pytest

from dense_fp32_matrix_row_amd import sgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hip_sgemm\w*)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(sgemm.EXPORTS)


@pytest.mark.parametrize("name", declared_functions())
def test_symbol_exported(name):
    lib = sgemm.load()
    assert hasattr(lib, name), name


def test_levels_and_names():
    n = sgemm.hip_sgemm_num_levels()
    assert n == 11
    names = [sgemm.hip_sgemm_level_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert names[0].startswith("L0_") and names[9].startswith("L9_mfma")
    assert names[10].startswith("L10_shape_dispatch")
    assert sgemm.hip_sgemm_level_name(-1) is None
    assert sgemm.hip_sgemm_level_name(n) is None


FAKE = 0x1000  # a non-NULL address that is never dereferenced (errors return first)


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4), -1),
    ((4, -1, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4), -2),
    ((4, 4, -1, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4), -3),
    ((4, 4, 4, 1.0, None, 4, FAKE, 4, 0.0, FAKE, 4), -5),
    ((4, 4, 8, 1.0, FAKE, 7, FAKE, 4, 0.0, FAKE, 4), -6),
    ((4, 4, 0, 1.0, FAKE, 0, FAKE, 4, 0.0, FAKE, 4), -6),    # lda >= max(1, K)
    ((4, 4, 4, 1.0, FAKE, 4, None, 4, 0.0, FAKE, 4), -7),
    ((4, 9, 4, 1.0, FAKE, 4, FAKE, 8, 0.0, FAKE, 9), -8),
    ((4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, None, 4), -10),
    ((4, 9, 4, 1.0, FAKE, 4, FAKE, 9, 0.0, FAKE, 8), -11),
    ((-1, -1, -1, 1.0, None, 0, None, 0, 0.0, None, 0), -1),  # first bad argument wins
])
def test_argument_errors(args, status):
    assert sgemm.hip_sgemm(*args, stream=0) == status
    for level in range(sgemm.hip_sgemm_num_levels()):
        assert sgemm.hip_sgemm_level(level, *args, stream=0) == status
    assert sgemm.hip_sgemm_status_string(status).startswith(f"argument {-status} ")


def test_null_operands_allowed_when_not_read():
    # M == 0 or N == 0: nothing is read or written, no launch -> success on CPU
    assert sgemm.hip_sgemm(0, 5, 5, 1.0, None, 5, None, 5, 0.0, None, 5, stream=0) == 0
    assert sgemm.hip_sgemm(5, 0, 5, 1.0, None, 5, None, 1, 0.0, None, 1, stream=0) == 0
    # alpha == 0: A and B may be NULL (validation passes; the check stops
    # before the launch by using M == 0)
    assert sgemm.hip_sgemm(0, 4, 4, 0.0, None, 4, None, 4, 1.0, None, 4, stream=0) == 0


def test_unknown_level():
    args = (4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4)
    assert sgemm.hip_sgemm_level(11, *args, stream=0) == sgemm.STATUS_UNKNOWN_LEVEL
    assert sgemm.hip_sgemm_level(-1, *args, stream=0) == sgemm.STATUS_UNKNOWN_LEVEL
    assert "unknown level" in sgemm.hip_sgemm_status_string(sgemm.STATUS_UNKNOWN_LEVEL)


def test_auto_level_is_the_dispatching_rung():
    for M, N, K in [(256, 256, 256), (4096, 4096, 4096), (4097, 4097, 4097), (1, 1, 1)]:
        assert sgemm.hip_sgemm_auto_level(M, N, K, FAKE, K, FAKE, N, FAKE, N) == 10
    assert sgemm.hip_sgemm_auto_level(-1, 2, 2, FAKE, 2, FAKE, 2, FAKE, 2) == -1


def test_launch_shapes():
    # level 9 picks its tile per problem: 256 x 128 for whole-tile large
    # problems, 128 x 128 (BK 32) mid-size, 128 x 64 large ragged, 64 x 64 small
    shape = sgemm.hip_sgemm_launch_shape(9, 4096, 4096, 4096)
    assert shape == {"workgroups": 512, "threads": 512, "k_steps": 256, "tile_m": 256, "tile_n": 128}
    shape = sgemm.hip_sgemm_launch_shape(9, 2048, 2048, 2048)
    assert shape == {"workgroups": 256, "threads": 256, "k_steps": 64, "tile_m": 128, "tile_n": 128}
    shape = sgemm.hip_sgemm_launch_shape(9, 4097, 4097, 4097)
    assert shape == {"workgroups": 33 * 65, "threads": 256, "k_steps": 257, "tile_m": 128, "tile_n": 64}
    shape = sgemm.hip_sgemm_launch_shape(9, 1024, 1024, 1024)
    assert shape == {"workgroups": 256, "threads": 256, "k_steps": 64, "tile_m": 64, "tile_n": 64}
    # level 10 reports its largest launch: the whole-tile grid of a problem
    # that misses the 256 x 128 tile by at most 16 rows / columns ...
    shape = sgemm.hip_sgemm_launch_shape(10, 4097, 4097, 4097)
    assert shape == {"workgroups": 512, "threads": 512, "k_steps": 257, "tile_m": 256, "tile_n": 128}
    shape = sgemm.hip_sgemm_launch_shape(10, 4096 + 16, 4096 + 16, 100)
    assert (shape["workgroups"], shape["tile_m"], shape["tile_n"]) == (512, 256, 128)
    # ... or the 128 x 128 tile (the assembly loop: 4 wavefronts, 16-deep
    # stages) when they fill whole rounds of CUs, or one round >= 70 % ...
    shape = sgemm.hip_sgemm_launch_shape(10, 2051, 2055, 300)
    assert shape == {"workgroups": 256, "threads": 256, "k_steps": 19, "tile_m": 128, "tile_n": 128}
    shape = sgemm.hip_sgemm_launch_shape(10, 2048, 4096, 2048)
    assert shape == {"workgroups": 512, "threads": 256, "k_steps": 128, "tile_m": 128, "tile_n": 128}
    shape = sgemm.hip_sgemm_launch_shape(10, 2048, 2048, 8192)
    assert shape == {"workgroups": 256, "threads": 256, "k_steps": 512, "tile_m": 128, "tile_n": 128}
    shape = sgemm.hip_sgemm_launch_shape(10, 1792, 1792, 1792)
    assert shape == {"workgroups": 196, "threads": 256, "k_steps": 112, "tile_m": 128, "tile_n": 128}
    # ... or, on a grid of >= 128 tiles of 64 x 64 (edge tiles partial), the
    # deep-stage 64 x 64 loop (4 K-slice wavefronts, 64-deep stages) ...
    for M, N, K in [(1024, 1024, 1024), (1536, 1536, 1536), (3072, 3072, 3072),
                    (1024, 1024, 4096), (768, 768, 768), (3000, 3000, 3000),
                    (4096 + 17, 4096, 64), (1000, 700, 300)]:
        shape = sgemm.hip_sgemm_launch_shape(10, M, N, K)
        assert shape == {"workgroups": -(-M // 64) * -(-N // 64), "threads": 256,
                         "k_steps": -(-K // 64), "tile_m": 64, "tile_n": 64}, (M, N, K)
    # ... split into K parts when K is deep and there is less than one round
    # of those tiles: at most two work items per CU (512 x 512 x 8192: 64
    # tiles in 8 parts of 1024) ...
    shape = sgemm.hip_sgemm_launch_shape(10, 512, 512, 8192)
    assert shape == {"workgroups": 64 * 8, "threads": 256, "k_steps": 16, "tile_m": 64, "tile_n": 64}
    # ... and otherwise (fewer than 128 such tiles, or 64 for a deep K) the thin
    # matrix-core kernel over 16-row panels: one block of 16 wavefronts per
    # panel and 16 columns, K in steps of 16 x 16
    for M, N, K in [(256, 256, 256), (300, 500, 100), (128, 512, 4096), (17, 300, 4096),
                    (512, 512, 512), (700, 500, 800)]:
        shape = sgemm.hip_sgemm_launch_shape(10, M, N, K)
        assert shape == {"workgroups": -(-M // 16) * -(-N // 16), "threads": 1024,
                         "k_steps": -(-K // 256), "tile_m": 16, "tile_n": 16}, (M, N, K)
    # ... and the thin kernels for M <= 16 (one block per 16 columns) or
    # N <= 16 (one block per 16 rows)
    shape = sgemm.hip_sgemm_launch_shape(10, 1, 4097, 4097)
    assert (shape["workgroups"], shape["threads"], shape["tile_n"]) == (257, 1024, 16)
    # (16 rows: the matrix-core form, 16 wavefronts per block of 16 columns)
    shape = sgemm.hip_sgemm_launch_shape(10, 16, 4096, 64)
    assert (shape["workgroups"], shape["threads"], shape["tile_m"], shape["tile_n"]) == (256, 1024, 16, 16)
    shape = sgemm.hip_sgemm_launch_shape(10, 16, 32768, 64)   # 64 columns per block
    assert (shape["workgroups"], shape["tile_n"]) == (512, 64)
    shape = sgemm.hip_sgemm_launch_shape(10, 8192, 8, 64)     # few columns: 32 rows per block
    assert (shape["workgroups"], shape["threads"], shape["tile_m"], shape["tile_n"]) == (256, 1024, 32, 16)
    shape = sgemm.hip_sgemm_launch_shape(10, 4096, 3, 4097)
    assert (shape["workgroups"], shape["threads"], shape["tile_m"], shape["tile_n"]) == (256, 1024, 16, 4)
    assert sgemm.hip_sgemm_launch_shape(2, 4096, 4096, 4096)["threads"] == 1024
    assert sgemm.hip_sgemm_launch_shape(0, 4096, 4096, 4096)["k_steps"] == 4096
    with pytest.raises(sgemm.SgemmError):
        sgemm.hip_sgemm_launch_shape(99, 1, 1, 1)


def test_phase_count_rounds_up_like_the_lecture_example():
    """Lecture 4 notes, section 8 exercise 6: K = 100 with 16-wide phases needs
    ceil(100/16) = 7 phases (the floor form would drop 4 terms).  Level 9
    stages BK = 16 and must walk exactly that many K steps; levels 7 and 8
    stage BK = 8 and round up the same way."""
    from tests.oracle_pins import golden
    g = golden()["phase_count"]
    shape = sgemm.hip_sgemm_launch_shape(9, 64, 64, g["K"])
    assert shape["k_steps"] == g["phases"]
    for level in (7, 8):
        assert sgemm.hip_sgemm_launch_shape(level, 64, 64, g["K"])["k_steps"] == -(-g["K"] // 8)
    assert sgemm.hip_sgemm_launch_shape(2, 64, 64, g["K"])["k_steps"] == -(-g["K"] // 32)


def test_tile32_geometry_matches_the_six_level_example():
    """SGEMM 六级优化, K3 section: with TILE = 32 the block at (x=2, y=3) owns
    C rows 96-127 x cols 64-95.  Level 2 uses the same 32 x 32 tile and 1024
    threads, so that block is tile (row 3, col 2) of its grid."""
    from tests.oracle_pins import golden
    g = golden()["tile32_block_thread"]
    shape = sgemm.hip_sgemm_launch_shape(2, 4096, 4096, 4096)
    assert shape["tile_m"] == shape["tile_n"] == g["tile"]
    assert shape["threads"] == g["tile"] * g["tile"]
    assert g["block_y"] * g["tile"] == g["block_rows"][0] and g["block_x"] * g["tile"] == g["block_cols"][0]
    assert (g["block_y"] * g["tile"] + g["ty"], g["block_x"] * g["tile"] + g["tx"]) == (g["c_row"], g["c_col"])
    coarse = golden()["coarse4_block"]
    assert sgemm.hip_sgemm_launch_shape(3, 4096, 4096, 4096)["tile_n"] == coarse["tile"] * coarse["coarse"]


def test_regtile8_cells_match_the_six_level_example():
    """SGEMM 六级优化, K4 section: the thread that computed C[103][69] in K3
    computes the eight cells C[96..103][69] of that column in K4.  Level 4
    is that kernel on 64 x 64 tiles: wavefront w of its 512 threads owns
    rows 8w .. 8w + 7 of the tile and lane l its column l (l4_regtile1d.hip),
    so the thread owning C[103][69] owns exactly the page's cells."""
    from tests.oracle_pins import golden
    g = golden()["regtile8_thread"]
    shape = sgemm.hip_sgemm_launch_shape(4, 4096, 4096, 4096)
    tm, tn, threads = shape["tile_m"], shape["tile_n"], shape["threads"]
    per_thread = tm * tn // threads
    assert per_thread == g["rows"][1] - g["rows"][0] + 1 == 8

    def cells(tile_row, tile_col, tid):
        w, lane = divmod(tid, tn)
        return [(tile_row * tm + per_thread * w + i, tile_col * tn + lane) for i in range(per_thread)]

    owners = [(tr, tc, tid) for tr in range(2) for tc in range(2) for tid in range(threads)
              if (103, 69) in cells(tr, tc, tid)]
    assert len(owners) == 1
    assert cells(*owners[0]) == [(r, g["col"]) for r in range(g["rows"][0], g["rows"][1] + 1)]


def test_tile_split_arguments():
    assert sgemm.hip_sgemm_num_tiles() == 17
    names = [sgemm.hip_sgemm_tile_name(t) for t in range(4)]
    assert names[0].startswith("256x128") and names[3].startswith("64x64")
    names = [sgemm.hip_sgemm_tile_name(t) for t in range(17)]
    assert names[4].startswith("128x128") and names[5].startswith("64x64") and "2slices" in names[5]
    assert names[6].startswith("64x64x64") and "4slices" in names[6]
    # the catalogue: every name states BM x BN x BK, all distinct
    assert all(n.startswith("cat_") for n in names[7:]) and len(set(names)) == 17
    for n in names:
        bm, bn, bk = (int(v) for v in n.removeprefix("cat_").split("_")[0].split("x"))
        assert bm % 64 == 0 and bn % 64 == 0 and bk in (16, 32, 64)
    assert sgemm.hip_sgemm_tile_name(17) is None and sgemm.hip_sgemm_tile_name(-1) is None
    args = (4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4)
    for tile, splits in [(-1, 1), (17, 1), (0, 0), (1, -3), (9, 0)]:
        assert sgemm.hip_sgemm_tile_split(tile, splits, *args, stream=0) == sgemm.STATUS_UNKNOWN_CONFIG
    assert "split" in sgemm.hip_sgemm_status_string(sgemm.STATUS_UNKNOWN_CONFIG)
    # argument errors as hip_sgemm once the configuration is valid
    assert sgemm.hip_sgemm_tile_split(0, 2, 4, 4, 8, 1.0, FAKE, 7, FAKE, 4, 0.0, FAKE, 4, stream=0) == -6
    assert sgemm.hip_sgemm_tile_split(1, 2, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, stream=0) == 0


@pytest.mark.parametrize("ops,args,status", [
    (("X", "N"), (4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4), sgemm.STATUS_BAD_OP_A),
    (("N", 2), (4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4), sgemm.STATUS_BAD_OP_B),
    (("N", "N"), (4, 4, 8, 1.0, FAKE, 7, FAKE, 4, 0.0, FAKE, 4), -6),
    (("T", "N"), (9, 4, 8, 1.0, FAKE, 8, FAKE, 4, 0.0, FAKE, 4), -6),   # A stored K x M: lda >= M
    (("T", "N"), (9, 4, 8, 1.0, FAKE, 9, FAKE, 4, 0.0, None, 4), -10),  # lda = M is fine
    (("N", "T"), (4, 9, 8, 1.0, FAKE, 8, FAKE, 7, 0.0, FAKE, 9), -8),   # B stored N x K: ldb >= K
    (("n", "t"), (4, 9, 8, 1.0, FAKE, 8, FAKE, 8, 0.0, None, 9), -10),  # ldb = K is fine
    (("C", "c"), (-1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4), -1),
    ((1, 0), (0, 4, 4, 1.0, None, 1, None, 4, 0.0, None, 4), 0),         # M == 0: nothing to do
])
def test_ex_argument_checks(ops, args, status):
    assert sgemm.hip_sgemm_ex(*ops, *args, stream=0) == status
    if status < -100:
        assert "op(" in sgemm.hip_sgemm_status_string(status)


def test_plan_query_names_every_plan_and_its_workspace():
    """hip_sgemm_plan says, before any call, which plan a shape takes, how
    many kernels it enqueues, and the split-K workspace (the only memory a
    call takes): S x M x N floats, S = ceil(K / slice)."""
    P = sgemm.hip_sgemm_plan
    assert P(0, 5, 5) == {"plan": 0, "name": "none", "launches": 0, "workspace_bytes": 0}
    assert P(5, 5, 0)["name"] == "scale"
    assert P(16, 4096, 4096)["name"] == "few_rows"
    assert P(4096, 3, 4097)["name"] == "few_cols"
    assert P(4096, 4096, 4096) == {"plan": 4, "name": "tiles", "launches": 1, "workspace_bytes": 0}
    # a fringe of one row and / or one column runs in the tiles' own launch
    # (every loop tile, on a grid with enough tiles for the blocks' shares);
    # wider fringes beside the 256 x 128 and 128 x 128 tiles add a
    # thin-kernel launch per side
    assert P(4097, 4097, 4097) == {"plan": 5, "name": "tiles_fringe", "launches": 1,
                                   "workspace_bytes": 0}
    assert P(4096, 4097, 64)["launches"] == 1 and P(4097, 4096, 64)["launches"] == 1
    assert P(4098, 4097, 64)["launches"] == 3 and P(4097, 4098, 64)["launches"] == 3
    assert P(4096, 4098, 64)["launches"] == 2
    for M, N, K, tile in [(2049, 2049, 2048, 128), (2049, 2048, 2048, 128), (1025, 1025, 1025, 64),
                          (1024, 1025, 1024, 64), (3073, 3073, 3073, 64), (1025, 4097, 37, 128),
                          (2561, 6145, 37, 256), (1025, 3073, 65, 64), (3073, 1024, 65, 64)]:
        assert P(M, N, K) == {"plan": 5, "name": "tiles_fringe", "launches": 1, "workspace_bytes": 0}
        g = sgemm.hip_sgemm_launch_shape(10, M, N, K)
        assert (g["tile_m"], g["workgroups"]) == (tile, (M // tile) * (N // g["tile_n"])), (M, N, K, g)
    assert P(2051, 2055, 300)["launches"] == 3  # 3 rows and 7 columns: thin kernels
    assert P(769, 769, 769)["name"] == "tiles"  # 12 x 12 tiles of 64 x 64: too few for the shares
    # 64 x 64 tiles take the fringe only where it leaves a CU fewer tiles
    # than the edge tiles would: 1537^3 has 576 whole tiles or 625 with
    # edges, three per CU either way
    assert P(1537, 1537, 1537)["name"] == "tiles"
    assert sgemm.hip_sgemm_launch_shape(10, 1537, 1537, 1537)["workgroups"] == 625
    assert P(256, 256, 256)["name"] == "thin_panels"
    # split K: 512 x 512 x 8192 (64 tiles of 64 x 64) in 8 slices of 1024
    sk = P(512, 512, 8192)
    assert sk["name"] == "split_k" and sk["launches"] == 2
    assert sk["workspace_bytes"] == 8 * 512 * 512 * 4
    # 700 x 600 x 8200: 110 tiles -> 4 slices of 2112 (a multiple of 64) -> 4 planes
    sk = P(700, 600, 8200)
    assert sk["name"] == "split_k" and sk["workspace_bytes"] == 4 * 700 * 600 * 4
    for M, N, K in [(4096, 4096, 4096), (1024, 1024, 1024), (100, 100, 100), (4097, 4097, 4097)]:
        assert P(M, N, K)["workspace_bytes"] == 0
    for bad, status in [((-1, 1, 1), -1), ((1, -1, 1), -2), ((1, 1, -1), -3)]:
        with pytest.raises(sgemm.SgemmError) as e:
            P(*bad)
        assert e.value.status == status


def test_split_k_workspace_bound_over_shapes():
    """Over a sweep of shapes, the split-K plan's workspace never exceeds
    512 tiles' worth of 64 x 64 planes (at most two work items per CU over
    256 CUs): 2^21 floats, 8 MiB."""
    worst = 0
    for M in range(64, 1100, 61):
        for N in range(64, 1100, 67):
            for K in (2048, 3000, 4096, 8192, 20000, 65536):
                info = sgemm.hip_sgemm_plan(M, N, K)
                if info["name"] == "split_k":
                    worst = max(worst, info["workspace_bytes"])
    assert 0 < worst <= 8 * 2 ** 20


def test_noalloc_argument_checks():
    """hip_sgemm_ex_noalloc validates like hip_sgemm_ex before touching the
    device: bad ops, BLAS argument positions, M == 0 quick return."""
    args = (4, 4, 8, 1.0, FAKE, 7, FAKE, 4, 0.0, FAKE, 4)
    assert sgemm.hip_sgemm_ex_noalloc("N", "N", *args, stream=0) == -6
    assert sgemm.hip_sgemm_ex_noalloc("Q", "N", *args, stream=0) == sgemm.STATUS_BAD_OP_A
    assert sgemm.hip_sgemm_ex_noalloc("N", 7, *args, stream=0) == sgemm.STATUS_BAD_OP_B
    assert sgemm.hip_sgemm_ex_noalloc("T", "N", 9, 4, 8, 1.0, FAKE, 8, FAKE, 4, 0.0, FAKE, 4,
                                      stream=0) == -6
    assert sgemm.hip_sgemm_ex_noalloc("N", "N", 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4,
                                      stream=0) == 0
    assert "fixed" in sgemm.hip_sgemm_status_string(sgemm.STATUS_WORKSPACE_LIMIT)


def test_load_with_a_path_serves_every_later_call(tmp_path):
    """sgemm.load(path) makes that build the module's library, so a caller
    comparing two builds in one process times the one it loaded."""
    import shutil
    copy = tmp_path / "libsgemm_copy.so"
    shutil.copy(sgemm.LIBRARY, copy)
    try:
        lib = sgemm.load(str(copy))
        assert sgemm.load() is lib and lib._name == str(copy)
        assert sgemm.hip_sgemm_num_levels() == 11
    finally:
        sgemm.load(sgemm.LIBRARY)
    assert sgemm.load()._name == sgemm.LIBRARY
