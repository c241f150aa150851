"""The test-side tiled-layout writer agrees with the FP6 E2M3 format
definition (CPU only)."""
import numpy as np

from tiling import e2m3, split_a6, tile


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
    codes[5, 0] = 1      # code 0 -> bits 0..5 of chunk 0, row 5
    codes[7, 33] = -7    # code 33 -> bits 198..203 -> chunk 3, bits 6..11
    t = tile(codes).reshape(6, 32, 8)
    assert t[0, 5, 0] == 0x08
    val = int.from_bytes(bytes(t[3, 7]), "little")
    assert (val >> 6) & 0x3F == 0x3E
    assert t.sum() == 0x08 + sum(bytes(t[3, 7]))


def test_a6_split():
    q = np.arange(-31, 32)
    qh, ql = split_a6(q)
    np.testing.assert_array_equal(8 * qh + ql, q)
    assert qh.min() >= -4 and qh.max() <= 3 and ql.min() >= 0 and ql.max() <= 7
