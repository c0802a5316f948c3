"""Host-side checks of the C ABI (CPU only: no HIP call is made).

The library must load without a GPU and export every function that
include/pgemm.h declares.  Argument checks, quick returns that touch nothing
(m == 0 or n == 0) and the variant choice all run before any HIP call, so
they are exercised here with placeholder addresses that are never
dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pgemm.h")

pg = pytest.importorskip("precision_gemm_02_amd", reason="libpgemm.so not built")
L = pg.library()
FAKE = 1 << 20          # 16-byte aligned placeholder address, never dereferenced
FAKE_ODD = FAKE + 4     # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_exports_every_declared_function():
    names = declared_functions()
    assert "gemm_f32" in names and "gemm_f64" in names and "matmat_f64" in names
    for name in names:
        assert hasattr(L, name), "libpgemm.so does not export %s" % name
    assert set(pg.EXPORTS) == set(names)


def f32(*a):
    return L.gemm_f32(*a)


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, None), -1),
    ((4, -1, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, None), -2),
    ((4, 4, -1, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, None), -3),
    ((4, 4, 4, 1.0, None, 4, FAKE, 4, 0.0, FAKE, 4, None), -5),
    ((4, 4, 4, 1.0, FAKE + 1, 4, FAKE, 4, 0.0, FAKE, 4, None), -5),   # misaligned
    ((4, 4, 4, 1.0, FAKE, 3, FAKE, 4, 0.0, FAKE, 4, None), -6),
    ((4, 4, 4, 1.0, FAKE, 4, None, 4, 0.0, FAKE, 4, None), -7),
    ((4, 4, 4, 1.0, FAKE, 4, FAKE, 3, 0.0, FAKE, 4, None), -8),
    ((4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, None, 4, None), -10),
    ((4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 3, None), -11),
    ((0, 4, 4, 1.0, FAKE, 0, FAKE, 4, 0.0, FAKE, 0, None), -6),        # lda >= 1 always
    ((4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, None), None),      # valid (not run)
])
def test_f32_argument_codes(args, code):
    if code is None:
        # a valid call would launch; check it through the selector instead
        assert pg.select_f32(*args[:11]) > 0
        return
    assert f32(*args) == code
    assert pg.select_f32(*args[:11]) == code


def test_first_bad_argument_wins():
    assert f32(-1, -1, -1, 1.0, None, 0, None, 0, 0.0, None, 0, None) == -1
    assert f32(4, 4, 4, 1.0, None, 1, None, 1, 0.0, None, 1, None) == -5


def test_f64_argument_codes():
    assert L.gemm_f64(4, 4, 4, ctypes.c_double(1.0), FAKE, 3, FAKE, 4, ctypes.c_double(0.0),
                      FAKE, 4, None) == -6
    assert L.gemm_f64(4, 4, 4, ctypes.c_double(1.0), FAKE + 4, 4, FAKE, 4,
                      ctypes.c_double(0.0), FAKE, 4, None) == -5


def test_quick_returns_touch_nothing():
    # m == 0 or n == 0: status 0 with NULL pointers and no HIP call
    assert f32(0, 5, 5, 1.0, None, 1, None, 5, 1.0, None, 1, None) == 0
    assert f32(5, 0, 5, 1.0, None, 5, None, 5, 1.0, None, 5, None) == 0
    assert L.gemm_f64(0, 0, 0, ctypes.c_double(1.0), None, 1, None, 1, ctypes.c_double(0.0),
                      None, 1, None) == 0


def test_null_ab_allowed_when_not_read():
    # k == 0 or alpha == 0: A and B may be NULL (selector: no GEMM kernel)
    assert pg.select_f32(4, 4, 0, 1.0, None, 4, None, 1, 2.0, FAKE, 4) == 0
    assert pg.select_f32(4, 4, 4, 0.0, None, 4, None, 4, 2.0, FAKE, 4) == 0


def test_matmat_argument_positions():
    mm = L.matmat_f64
    ok = (8, 8, 8, FAKE, FAKE, FAKE, 8, 8, 8, None)
    for pos, bad in ((1, 7), (2, 7), (3, 7)):
        args = list(ok)
        args[pos - 1] = bad
        assert mm(*args) == -pos
    args = list(ok); args[3] = None; assert mm(*args) == -4
    args = list(ok); args[4] = None; assert mm(*args) == -5
    args = list(ok); args[5] = None; assert mm(*args) == -6
    args = list(ok); args[6] = -1; assert mm(*args) == -7
    args = list(ok); args[7] = -1; args[0] = 8; assert mm(*args) == -8
    args = list(ok); args[8] = -1; args[1] = 8; args[2] = 8; assert mm(*args) == -9
    assert mm(8, 8, 8, None, None, None, 0, 8, 8, None) == 0


def test_variant_names_and_ids():
    names = pg.variants()
    assert len(names) == L.pgemm_num_variants() >= 4
    assert all(n.startswith("f32_") or n.startswith("f64_") for n in names.values())
    assert L.pgemm_variant_name(0) is None
    assert L.pgemm_variant_name(len(names) + 1) is None
    f64_id = min(v for v, n in names.items() if n.startswith("f64_"))
    assert L.gemm_f32_variant(f64_id, 4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, None) \
        == pg.PGEMM_EVARIANT


def name_of(v):
    return pg.variants()[v]


def test_selection_by_shape_and_alignment():
    # large square: 256 x 256 tiles; 2048: 128 x 128 tiles (256 tiles fill 256 CUs)
    v = pg.select_f32(8192, 8192, 8192, 1.5, FAKE, 8192, FAKE, 8192, 0.5, FAKE, 8192)
    assert name_of(v).startswith("f32_256x256") and name_of(v).endswith("_vec")
    v = pg.select_f32(2048, 2048, 2048, 1.0, FAKE, 2048, FAKE, 2048, 0.0, FAKE, 2048)
    assert name_of(v).startswith("f32_128x128") and name_of(v).endswith("_vec")
    # 1024^2: 256 tiles of 64 x 64
    v = pg.select_f32(1024, 1024, 1024, 1.0, FAKE, 1024, FAKE, 1024, 0.0, FAKE, 1024)
    assert name_of(v) == "f32_64x64x16_w2x2_s4_vec"
    # the same tiles with a long K loop: two K groups of 4 waves per tile
    v = pg.select_f32(1024, 1024, 8192, 1.0, FAKE, 1024, FAKE, 8192, 0.0, FAKE, 1024)
    assert name_of(v) == "f32_64x64x32_w2x2_s3_k2_vec"
    v = pg.select_f32(1024, 1024, 8192, 1.0, FAKE_ODD, 1024, FAKE, 8192, 0.0, FAKE, 1024)
    assert name_of(v) == "f32_64x64x32_w2x2_s3_k2_ua"
    # 32 x 32 tiles in four K groups: small problems, and up to three tiles
    # per compute unit, which run together (640^3: 400 tiles; 768^3: 576);
    # four or more per unit are priced in groups of three per unit, which
    # still leaves 896^3 (784 tiles) and 1024^3 (1024) to 64 x 64 tiles
    for n in (128, 512, 640, 768):
        v = pg.select_f32(n, n, n, 1.0, FAKE, n, FAKE, n, 0.0, FAKE, n)
        assert name_of(v) == "f32_32x32x64_w1x1_s3_k4_vec", (n, name_of(v))
    v = pg.select_f32(896, 896, 896, 1.0, FAKE, 896, FAKE, 896, 0.0, FAKE, 896)
    assert name_of(v) == "f32_64x64x16_w2x2_s4_vec"
    # 4 to 9 of them per unit with K loops of 12 K tiles or more are priced in
    # groups of three per unit: 1152^3 (1296 tiles) and 1100 x 1000 x 900 run
    # as 32 x 32 tiles (measured 10-16 % faster than 64 x 64); ~20 per unit
    # (2924 x 1760 x 4292) or 8 K tiles (3192 x 460 x 516) keep larger tiles
    for e in ((1152, 1152, 1152), (1100, 1000, 900)):
        v = pg.select_f32(*e, 1.0, FAKE, e[0], FAKE, e[2], 0.0, FAKE, e[0])
        assert name_of(v) == "f32_32x32x64_w1x1_s3_k4_vec", (e, name_of(v))
    for e in ((2924, 1760, 4292), (3192, 460, 516)):
        v = pg.select_f32(*e, 1.0, FAKE, e[0], FAKE, e[2], 0.0, FAKE, e[0])
        assert not name_of(v).startswith("f32_32x32"), (e, name_of(v))
    # one such tile per unit with a long K loop is priced low enough that
    # stream-K of 64 x 64 tiles takes it where a workspace allows
    e = (732, 316, 3260, 1.0, FAKE, 732, FAKE, 3260, 0.0, FAKE, 732)
    assert name_of(pg.select_f32(*e)) == "f32_32x32x64_w1x1_s3_k4_vec"
    v, sk, _ = pg.select_ws_f32(*e, pg.workspace_f32(*e[:3]))
    assert name_of(v) == "f32_64x64x16_w2x2_s4_vec" and sk > 0
    # odd leading dimensions select the unaligned path
    v = pg.select_f32(4097, 3001, 1023, 0.75, FAKE, 4113, FAKE, 1039, -1.25, FAKE, 4113)
    assert name_of(v).endswith("_ua")
    # a 4-byte aligned pointer selects the unaligned path
    v = pg.select_f32(512, 512, 512, 1.0, FAKE_ODD, 512, FAKE, 512, 0.0, FAKE, 512)
    assert name_of(v).endswith("_ua")
    v = pg.select_f64(4096, 4096, 4096, 1.0, FAKE, 4104, FAKE, 4104, 1.0, FAKE, 4104)
    assert name_of(v).startswith("f64_") and name_of(v).endswith("_vec")
    v = pg.select_f64(100, 100, 100, 1.0, FAKE, 101, FAKE, 100, 1.0, FAKE, 100)
    assert name_of(v).endswith("_ua")


def test_64x64_class_ldc_limit():
    """The 64 x 64 tiles (fp32 with one or two K groups, fp64) store C through
    a buffer descriptor at a tile's first element with 32-bit byte offsets,
    which hold 64 columns of ldc up to 8388606 fp32 or 4194302 fp64 elements.  Beyond that the planner takes another class (with and
    without a workspace), and the forced variant is refused before any
    launch."""
    lim = 8388606
    v = pg.select_f32(1024, 1024, 1024, 1.0, FAKE, 1024, FAKE, 1024, 0.0, FAKE, lim - 2)
    assert name_of(v) == "f32_64x64x16_w2x2_s4_vec"
    for ldc in (lim + 2, 1 << 24):
        v = pg.select_f32(1024, 1024, 1024, 1.0, FAKE, 1024, FAKE, 1024, 0.0, FAKE, ldc)
        assert not name_of(v).startswith("f32_64x64x16"), (ldc, name_of(v))
        e = (732, 316, 3260, 1.0, FAKE, 732, FAKE, 3260, 0.0, FAKE, ldc)
        v, _, _ = pg.select_ws_f32(*e, pg.workspace_f32(*e[:3]))
        assert not name_of(v).startswith("f32_64x64x16"), (ldc, name_of(v))
    ids = {n: v for v, n in pg.variants().items()}
    for name in ("f32_64x64x16_w2x2_s4_vec", "f32_64x64x16_w2x2_s4_ua"):
        assert L.gemm_f32_variant(ids[name], 1024, 1024, 1024, 1.0, FAKE, 1024, FAKE, 1024,
                                  0.0, FAKE, lim + 2, None) == pg.PGEMM_EVARIANT
    # the two-K-group 64 x 64 class stores C the same way
    v = pg.select_f32(1024, 1024, 8192, 1.0, FAKE, 1024, FAKE, 8192, 0.0, FAKE, lim - 2)
    assert name_of(v) == "f32_64x64x32_w2x2_s3_k2_vec"
    v = pg.select_f32(1024, 1024, 8192, 1.0, FAKE, 1024, FAKE, 8192, 0.0, FAKE, 1 << 24)
    assert not name_of(v).startswith("f32_64x64"), name_of(v)
    for name in ("f32_64x64x32_w2x2_s3_k2_vec", "f32_64x64x32_w2x2_s3_k2_ua"):
        assert L.gemm_f32_variant(ids[name], 1024, 1024, 8192, 1.0, FAKE, 1024, FAKE, 8192,
                                  0.0, FAKE, lim + 2, None) == pg.PGEMM_EVARIANT
    # other classes take any ldc
    v = pg.select_f32(2048, 2048, 2048, 1.0, FAKE, 2048, FAKE, 2048, 0.0, FAKE, 1 << 24)
    assert name_of(v).startswith("f32_128x128")
    # fp64 64 x 64 tiles: 64 columns of 8-byte elements, ldc up to 4194302
    lim64 = 4194302
    v = pg.select_f64(1024, 1024, 1024, 1.0, FAKE, 1024, FAKE, 1024, 1.0, FAKE, lim64)
    assert name_of(v) == "f64_64x64x16_w2x4_s4_vec"
    v = pg.select_f64(1024, 1024, 1024, 1.0, FAKE, 1024, FAKE, 1024, 1.0, FAKE, lim64 + 2)
    assert not name_of(v).startswith("f64_64x64"), name_of(v)
    assert L.gemm_f64_variant(ids["f64_64x64x16_w2x4_s4_ua"], 1024, 1024, 1024,
                              ctypes.c_double(1.0), FAKE, 1024, FAKE, 1024, ctypes.c_double(1.0),
                              FAKE, lim64 + 1, None) == pg.PGEMM_EVARIANT


def test_selection_with_workspace():
    # 2150 x 2030 x 1000: with the workspace it asks for, 128 x 128 tiles (a
    # full round of 256 + 16) with 240 stream-K workgroups (15 per leftover
    # tile: no range crosses a tile); without it, or with one byte less, the
    # plain choice (no stream-K)
    args = (2150, 2030, 1000, 0.75, FAKE, 2151, FAKE, 1001, -1.25, FAKE, 2153)
    ws = pg.workspace_f32(*args[:3])
    v, sk, strip = pg.select_ws_f32(*args, ws)
    assert name_of(v) == "f32_128x128x16_w4x2_s4_ua" and sk == 240 and strip == 0
    for short in (0, ws - 1):
        v0, sk0, strip0 = pg.select_ws_f32(*args, short)
        assert v0 == pg.select_f32(*args) and sk0 == 0 and strip0 == 0
    # the ragged 4097 x 3001 x 1023 problem: row 4097 goes to the strip
    # kernel and 128 x 128 tiles fill 3 rounds exactly, with or without a
    # workspace (it asks for none)
    args = (4097, 3001, 1023, 0.75, FAKE, 4113, FAKE, 1039, -1.25, FAKE, 4113)
    assert pg.workspace_f32(*args[:3]) == 0
    v, sk, strip = pg.select_ws_f32(*args, 0)
    assert name_of(v) == "f32_128x128x16_w4x2_s4_ua" and sk == 0 and strip == 1
    assert v == pg.select_f32(*args)
    # shapes that fill whole rounds: same as the plain entry point
    sq = (8192, 8192, 8192, 1.5, FAKE, 8192, FAKE, 8192, 0.5, FAKE, 8192)
    assert pg.select_ws_f32(*sq, 1 << 30) == (pg.select_f32(*sq), 0, 0)
    d = (4096, 4096, 4096, 1.0, FAKE, 4104, FAKE, 4104, 1.0, FAKE, 4104)
    assert pg.select_ws_f64(*d, 1 << 30) == (pg.select_f64(*d), 0, 0)
    # 8 leftover 128 x 128 tiles of 50 K tiles: 12 workgroups per tile (each
    # keeps at least 4 K tiles) -> 96, no range crossing a tile
    e = (725, 5528, 796, 1.0, FAKE, 725, FAKE, 796, 1.0, FAKE, 725)
    v, sk, _ = pg.select_ws_f32(*e, pg.workspace_f32(*e[:3]))
    assert name_of(v).startswith("f32_128x128") and sk == 96
    # 129 leftover tiles (above half the units): all 256 units, ranges of
    # 35-36 K tiles that cross tiles
    e = (1351, 4463, 1130, 1.0, FAKE, 1351, FAKE, 1130, 1.0, FAKE, 1351)
    v, sk, _ = pg.select_ws_f32(*e, pg.workspace_f32(*e[:3]))
    assert name_of(v).startswith("f32_128x128") and sk == 256
    # thin shapes with long K loops: 64 x 64 tiles with two K groups, whose
    # stream-K form shares the partly filled last round (256 + 23 tiles of 92
    # K tiles over 253 workgroups; 64 tiles, no full round, of 256 K tiles
    # over 256)
    e = (5933, 138, 2931, 1.0, FAKE, 5936, FAKE, 2932, 1.0, FAKE, 5936)
    v, sk, _ = pg.select_ws_f32(*e, pg.workspace_f32(*e[:3]))
    assert name_of(v) == "f32_64x64x32_w2x2_s3_k2_vec" and sk == 253
    e = (2047, 96, 8191, 1.0, FAKE, 2051, FAKE, 8193, 1.0, FAKE, 2051)
    v, sk, _ = pg.select_ws_f32(*e, pg.workspace_f32(*e[:3]))
    assert name_of(v) == "f32_64x64x32_w2x2_s3_k2_ua" and sk == 256
    # where two or three 32 x 32 tiles share each compute unit they run
    # together, which beats stream-K of 64 x 64 tiles (3000 x 160 x 4000:
    # 470 tiles; measured 40.6 against 64.7 us)
    e = (3000, 160, 4000, 1.0, FAKE, 3000, FAKE, 4000, 1.0, FAKE, 3000)
    v, sk, _ = pg.select_ws_f32(*e, pg.workspace_f32(*e[:3]))
    assert name_of(v) == "f32_32x32x64_w1x1_s3_k4_vec" and sk == 0
    # invalid arguments: the same status as the plain selector, no stream-K
    bad = (4, 4, 4, 1.0, FAKE, 3, FAKE, 4, 0.0, FAKE, 4)
    assert pg.select_ws_f32(*bad, 1 << 20) == (-6, 0, 0)


def test_plan_invariants_on_random_shapes():
    """Host logic only: for seeded random shapes, the plan the workspace
    entry point reports is consistent with the tiling it names (256 compute
    units, the fallback without a GPU): the workspace holds two tiles of
    partial sums per stream-K workgroup; stream-K workgroups outnumber the
    leftover tiles, at most one per compute unit, each with at least 4 K
    tiles after a full round (2 without one); strip rows are the 1 to 8 rows
    below whole tile rows; without a workspace the choice is the plain one."""
    rng = np.random.default_rng(8)
    for t in range(400):
        f32 = t % 3 != 0
        m, n = (int(x) for x in rng.integers(1, 9000, 2))
        k = int(rng.integers(1, 4000))
        sel = pg.select_ws_f32 if f32 else pg.select_ws_f64
        plain = pg.select_f32 if f32 else pg.select_f64
        size = 4 if f32 else 8
        args = (m, n, k, 1.0, FAKE, m, FAKE, k, 0.0, FAKE, m)
        ws = (pg.workspace_f32 if f32 else pg.workspace_f64)(m, n, k)
        v, sk, strip = sel(*args, ws)
        bm, bn, bk = (int(x) for x in re.match(r"f\d\d_(\d+)x(\d+)x(\d+)", name_of(v)).groups())
        if strip:
            assert 1 <= strip <= 8 and (m - strip) % bm == 0 and m > bm, (m, n, k, strip)
        tiles = -(-(m - strip) // bm) * -(-n // bn)
        rest = tiles % 256
        if sk:
            assert ws == 2 * sk * bm * bn * size
            assert rest > 0 and rest < sk <= 256, (m, n, k, sk, rest)
            assert rest * -(-k // bk) // sk >= (4 if tiles >= 256 else 2)
        else:
            assert ws == 0
        v0, sk0, strip0 = sel(*args, 0)
        assert v0 == plain(*args) and sk0 == 0


def test_device_info_argument_codes():
    out = ctypes.c_int(0)
    assert L.pgemm_device_info(None, ctypes.byref(out)) == -1
    assert L.pgemm_device_info(ctypes.byref(out), None) == -2


def test_status_strings():
    assert pg.status_string(0) == "success"
    assert "launch" in pg.status_string(pg.PGEMM_EHIP)
    assert "invalid argument" in pg.status_string(-6)
    assert pg.status_string(12345) == "unknown status"


def test_binding_raises_on_bad_status():
    with pytest.raises(pg.PgemmError) as e:
        pg.gemm_f32(4, 4, 4, 1.0, FAKE, 3, FAKE, 4, 0.0, FAKE, 4, stream=0)
    assert e.value.status == -6


def test_workspace_entry_points_host_checks():
    ws32 = L.gemm_f32_ws
    # ordinary argument errors keep their positions; a workspace that is not
    # 16-byte aligned is argument 12
    assert ws32(4, 4, 4, 1.0, FAKE, 3, FAKE, 4, 0.0, FAKE, 4, None, 0, None) == -6
    assert ws32(4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, FAKE + 4, 1 << 20, None) == -12
    assert L.gemm_f64_ws(4, 4, 4, ctypes.c_double(1.0), FAKE, 4, FAKE, 4,
                         ctypes.c_double(0.0), FAKE, 4, FAKE + 8, 1 << 20, None) == -12
    # quick return with no memory touched
    assert ws32(0, 4, 4, 1.0, None, 1, None, 4, 0.0, None, 1, None, 0, None) == 0


def test_workspace_sizes():
    # 8192^3: 1024 tiles of 256 x 256 fill whole rounds on 256 CUs -> none
    assert pg.workspace_f32(8192, 8192, 8192) == 0
    assert pg.workspace_f32(2048, 2048, 2048) == 0
    assert pg.workspace_f32(0, 10, 10) == 0 and pg.workspace_f32(10, 10, 0) == 0
    # 2150 x 2030 x 1000 on 128 x 128 x 16 tiles: 17 x 16 = 272 tiles = a
    # round of 256 + 16 leftover tiles (63 K tiles each) shared by 240
    # workgroups, two workspace slots each.  256 compute units: the MI355X,
    # and the fallback with no GPU.
    assert pg.workspace_f32(2150, 2030, 1000) == 2 * 240 * 128 * 128 * 4
    # 4097 x 3001 x 1023: the strip kernel takes the last row, and the tiles
    # of the other 4096 fill 3 rounds: no workspace
    assert pg.workspace_f32(4097, 3001, 1023) == 0
    # 3840^3: 900 tiles of 128^2 = 3 rounds + 132, a last round above half
    # full, still shared
    assert pg.workspace_f32(3840, 3840, 3840) == 2 * 256 * 128 * 128 * 4
    assert pg.workspace_f64(3840, 3840, 3840) == 2 * 256 * 128 * 128 * 8
    # too few K tiles to share after a full round (4 per workgroup)
    assert pg.workspace_f32(4097, 3001, 100) == 0
    # 512^3 fp32: 64 tiles of 64^2; sharing them is estimated not to pay for
    # the fix-up kernel's launch
    assert pg.workspace_f32(512, 512, 512) == 0
    # 1024^3 is one round of 256 such tiles: none
    assert pg.workspace_f32(1024, 1024, 1024) == 0
    # 74 x 104 x 771 fp64: 4 tiles of 64^2 with 49 K tiles, 24 workgroups per
    # tile (at least 2 K tiles each) -> 96 workgroups
    assert pg.workspace_f64(74, 104, 771) == 2 * 96 * 64 * 64 * 8


def test_matmat_host_argument_codes_and_quick_returns():
    mm = L.matmat_f64_host
    ws = FAKE
    need = pg.matmat_host_workspace(8, 8, 8, 8, 8, 8)
    ok = [8, 8, 8, FAKE, FAKE, FAKE, 8, 8, 8, ws, need, None]
    for pos, bad in ((1, 7), (2, 7), (3, 7)):
        args = list(ok)
        args[pos - 1] = bad
        assert mm(*args) == -pos
    for pos in (4, 5, 6):
        args = list(ok)
        args[pos - 1] = None
        assert mm(*args) == -pos
    args = list(ok); args[9] = None; assert mm(*args) == -10
    args = list(ok); args[9] = FAKE + 8; assert mm(*args) == -10    # not 16-byte aligned
    args = list(ok); args[10] = need - 1; assert mm(*args) == -11
    # empty C, or N2 = 0 (C + A*B = C): nothing touched, no workspace needed
    assert mm(8, 8, 8, None, None, None, 0, 8, 8, None, 0, None) == 0
    assert mm(1, 8, 8, None, None, FAKE, 8, 0, 8, None, 0, None) == 0


def test_matmat_host_workspace_size():
    # strided blocks ((rows-1)*ld + cols doubles), each rounded up to 256 bytes
    def r256(b):
        return (b + 255) // 256 * 256
    for (lda, ldb, ldc, n1, n2, n3) in ((8, 8, 8, 8, 8, 8), (6, 4, 9, 7, 5, 3),
                                        (4104, 4104, 4104, 4096, 4096, 4096), (1, 1, 1, 1, 1, 1)):
        want = (r256(((n1 - 1) * lda + n2) * 8) + r256(((n2 - 1) * ldb + n3) * 8)
                + r256(((n1 - 1) * ldc + n3) * 8))
        assert pg.matmat_host_workspace(lda, ldb, ldc, n1, n2, n3) == want
    assert pg.matmat_host_workspace(5, 5, 5, 0, 5, 5) == 0
    assert pg.matmat_host_workspace(4, 5, 5, 5, 5, 5) == 0    # lda < N2


def test_cpu_tensors_are_refused_before_any_call(monkeypatch):
    """A CPU tensor's data pointer is a host address: handed to a kernel it
    would fault the GPU.  The binding refuses it with TypeError before the
    library is called (the library is replaced by one that records calls)."""
    import torch
    calls = []

    class Rec:
        def __getattr__(self, name):
            def f(*a):
                calls.append(name)
                return 0
            return f

    monkeypatch.setattr(pg, "_lib", Rec())
    A = torch.zeros(8, 8)
    B = torch.zeros(8, 8)
    C = torch.zeros(8, 8)
    with pytest.raises(TypeError):
        pg.gemm_f32(8, 8, 8, 1.0, A, 8, B, 8, 0.0, C, 8, stream=0)
    with pytest.raises(TypeError):
        pg.gemm_f64(8, 8, 8, 1.0, A.double(), 8, B.double(), 8, 0.0, C.double(), 8, stream=0)
    with pytest.raises(TypeError):
        pg.matmat_f64(8, 8, 8, A.double(), B.double(), C.double(), 8, 8, 8, stream=0)
    with pytest.raises(TypeError):
        pg.gemm_f32_ws(8, 8, 8, 1.0, FAKE, 8, FAKE, 8, 0.0, FAKE, 8,
                       torch.zeros(16, dtype=torch.uint8), 16, stream=0)
    with pytest.raises(TypeError):
        pg.gemm(A, B, C)
    with pytest.raises(TypeError):
        pg.gemm_f32(8, 8, 8, 1.0, "not a pointer", 8, FAKE, 8, 0.0, FAKE, 8, stream=0)
    assert calls == []
    # integer device addresses pass through unchanged (the caller vouches)
    pg.gemm_f32(8, 8, 8, 1.0, FAKE, 8, FAKE, 8, 0.0, FAKE, 8, stream=0)
    assert calls == ["gemm_f32"]


def test_layouts_of_vectors_fit_both():
    """_layouts: a dimension of size 1 fits column- and row-major alike, so
    matrix-vector and outer products of contiguous (row-major) or
    column-major tensors find one common layout."""
    import torch
    L_ = pg._layouts
    # contiguous (row-major) A (m x k), B (k x 1), C (m x 1): n == 1
    assert L_(torch.empty(5, 3)) == {"row": 3}
    assert L_(torch.empty(3, 1)) == {"col": 3, "row": 1}
    # k == 1: A (m x 1), B (1 x n)
    assert L_(torch.empty(1, 4)) == {"col": 1, "row": 4}
    # column-major views
    assert L_(torch.empty(3, 5).t()) == {"col": 5}
    assert L_(torch.empty(1, 5).t()) == {"col": 5, "row": 1}
    # padded column-major: ld from the stride
    assert L_(torch.empty(4, 10).t()[:7, :]) == {"col": 10}
    assert L_(torch.empty(1, 1)) == {"col": 1, "row": 1}
    with pytest.raises(ValueError):
        L_(torch.empty(4, 6)[:, ::2])
    with pytest.raises(ValueError):
        L_(torch.empty(2, 3, 4))
    # every combination of a matrix-vector call shares a layout
    for (m, k, n) in ((5, 3, 1), (5, 1, 4), (1, 3, 4), (1, 1, 1)):
        la, lb, lc = L_(torch.empty(m, k)), L_(torch.empty(k, n)), L_(torch.empty(m, n))
        assert "row" in la and "row" in lb and "row" in lc
        la, lb, lc = (L_(torch.empty(c, r).t()) for (r, c) in ((m, k), (k, n), (m, n)))
        assert "col" in la and "col" in lb and "col" in lc


def test_noalloc_host_checks_and_scratch_bound():
    """gemm_f32_noalloc: argument codes in gemm_f32's positions and quick
    returns before any HIP call; the scratch size the header states is the
    binding's; and on 256 compute units (the MI355X, and the fallback without
    a GPU) no fp32 shape's stream-K workspace exceeds it, so the call never
    returns PGEMM_ESCRATCH there."""
    nf = L.gemm_f32_noalloc
    assert nf(4, 4, 4, 1.0, FAKE, 3, FAKE, 4, 0.0, FAKE, 4, None) == -6
    assert nf(4, 4, 4, 1.0, None, 4, FAKE, 4, 0.0, FAKE, 4, None) == -5
    assert nf(-1, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4, None) == -1
    assert nf(0, 5, 5, 1.0, None, 1, None, 5, 1.0, None, 1, None) == 0
    hdr = open(HEADER).read()
    m = re.search(r"#define PGEMM_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and (int(m.group(1)) << int(m.group(2))) == pg.PGEMM_SCRATCH_BYTES
    assert "scratch" in pg.status_string(pg.PGEMM_ESCRATCH)
    rng = np.random.default_rng(11)
    worst = 0
    for _ in range(3000):
        m_, n_ = (int(x) for x in rng.integers(1, 12000, 2))
        k_ = int(rng.integers(1, 9000))
        worst = max(worst, pg.workspace_f32(m_, n_, k_))
    assert 0 < worst <= pg.PGEMM_SCRATCH_BYTES
    # the largest plan: 256 stream-K workgroups of 128 x 128 tiles
    assert pg.workspace_f32(3840, 3840, 3840) == pg.PGEMM_SCRATCH_BYTES
