"""The test-side tiled-layout writer agrees with the FP6 E2M3 format
definition (CPU only)."""
import numpy as np

from tiling import e2m3, row_mask, row_mask_mx, split_a6, tile, tile_mx


def _decode_e2m3(f):
    f = np.asarray(f, dtype=np.int64)
    s, e, m = (f >> 5) & 1, (f >> 3) & 3, f & 7
    v = np.where(e == 0, m / 8.0, (1 + m / 8.0) * 2.0 ** (e - 1))
    return np.where(s == 1, -v, v)


def test_e2m3_exact_for_int4_codes():
    q = np.arange(-7, 8)
    np.testing.assert_array_equal(_decode_e2m3(e2m3(q)), q)


def test_tile_bit_placement():
    codes = np.zeros((32, 64), dtype=np.int64)
    codes[5, 0] = 1      # row 5, half 0, code 0 -> bits 0..5 of lane 5's string (byte 16*5)
    codes[7, 33] = -7    # row 7, half 1, code 1 -> bits 6..11 of lane 39's string
    codes[2, 31] = 2     # row 2, half 0, code 31 -> bits 186..191 -> byte 23 -> tail byte 7 of lane 2
    t = tile(codes)
    assert t[16 * 5] == 0x08
    val = int.from_bytes(bytes(t[16 * 39:16 * 39 + 2]), "little")
    assert (val >> 6) & 0x3F == 0x3E
    assert t[1024 + 8 * 2 + 7] == (0x10 << 2) & 0xFF      # 2 -> 0x10 in E2M3, bits 2..7 of byte 23
    assert int(t.sum()) == 0x08 + sum(bytes(t[16 * 39:16 * 39 + 2])) + ((0x10 << 2) & 0xFF)


def test_row_mask():
    m = row_mask(40, 128).reshape(2, 2, 1536)
    assert m[0].all()                                 # rows 0..31 all live
    assert m[1, :, 16 * 7].all() and not m[1, :, 16 * 8].any()        # row 39 live, row 40 not (half 0)
    assert m[1, :, 16 * (32 + 7)].all() and not m[1, :, 16 * (32 + 8)].any()
    assert m[1, :, 1024 + 8 * 7].all() and not m[1, :, 1024 + 8 * 8].any()


def test_a6_split():
    q = np.arange(-31, 32)
    qh, ql = split_a6(q)
    np.testing.assert_array_equal(8 * qh + ql, q)
    assert qh.min() >= -4 and qh.max() <= 3 and ql.min() >= 0 and ql.max() <= 7


def test_tile_mx_placement():
    R, K = 40, 256
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    e8 = np.full((R, K // 32), 127, dtype=np.uint8)
    codes[33, 80] = 0xA5        # row 33 (block 1, r 1), k = 160..161: kg 2, half 1, byte 0 of its 16
    e8[33, 5] = 130             # block 5 -> k-slice 1, byte 1
    t, s = tile_mx(codes, e8)
    G, Rp = K // 64, 64
    assert t.size == Rp * K // 2 and s.size == Rp * K // 32
    off = (1 * G + 2) * 1024 + 16 * (32 * 1 + 1)
    assert t[off] == 0xA5 and int(t.sum()) == 0xA5
    assert s[(1 * Rp + 33) * 4 + 1] == 130
    assert np.count_nonzero(s != 127) == 1
    m = row_mask_mx(R, K).reshape(Rp // 32, G, 2, 32, 16)
    assert m[1, :, :, 7].all() and not m[1, :, :, 8].any()



def test_layout_readers_invert_the_writers():
    from tiling import tile, tile_mx, untile, untile_mx
    rng = np.random.default_rng(21)
    q = rng.integers(-7, 8, size=(70, 256))
    np.testing.assert_array_equal(untile(tile(q), 70, 256), q)
    c = rng.integers(0, 256, size=(45, 128)).astype(np.uint8)
    e = rng.integers(0, 256, size=(45, 8)).astype(np.uint8)
    tc, ts = tile_mx(c, e)
    c2, e2 = untile_mx(tc, ts, 45, 256)
    np.testing.assert_array_equal(c2, c)
    np.testing.assert_array_equal(e2, e)
