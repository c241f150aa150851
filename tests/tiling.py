"""NumPy writer of the tiled FP6 operand layout, from its definition in
include/oq.h (a data layout, no arithmetic of the method): rows padded to 32,
the 64 codes of (row r, k-group kg) form a 384-bit string with code j in bits
[6j, 6j+6); chunk c (8 bytes) of it sits at
((r/32) * (K/64) + kg) * 1536 + c * 256 + (r % 32) * 8.
FP6 E2M3: sign bit 5, exponent bits 4..3 (bias 1), mantissa bits 2..0."""
import numpy as np

# E2M3 bit patterns of the integers 0..7, written from the format definition:
# 1 = 2^0 (e=1, m=0), 2 = 2^1 (e=2), 3 = 2^1 * 1.5 (e=2, m=4), 4 = 2^2 (e=3),
# 5 = 2^2 * 1.25 (m=2), 6 = 2^2 * 1.5 (m=4), 7 = 2^2 * 1.75 (m=6)
E2M3_OF_INT = np.array([0x00, 0x08, 0x10, 0x14, 0x18, 0x1A, 0x1C, 0x1E], dtype=np.uint64)


def e2m3(q):
    q = np.asarray(q, dtype=np.int64)
    assert np.all(np.abs(q) <= 7)
    return E2M3_OF_INT[np.abs(q)] | np.where(q < 0, np.uint64(0x20), np.uint64(0))


def tile(codes: np.ndarray) -> np.ndarray:
    """int codes [R, K] in [-7, 7] -> tiled bytes (R padded to 32)."""
    R, K = codes.shape
    assert K % 64 == 0
    Rp = (R + 31) // 32 * 32
    G = K // 64
    c = np.zeros((Rp, K), dtype=np.int64)
    c[:R] = codes
    f = e2m3(c).reshape(Rp, G, 64)
    out = np.zeros((Rp // 32, G, 6, 32, 8), dtype=np.uint8)
    for j in range(64):
        bit = 6 * j
        for b in range(6):
            pos = bit + b
            chunk, inchunk = pos // 64, pos % 64
            byte, bitpos = inchunk // 8, inchunk % 8
            v = ((f[:, :, j] >> np.uint64(b)) & np.uint64(1)).astype(np.uint8)  # [Rp, G]
            out[:, :, chunk, :, byte] |= (v.reshape(Rp // 32, 32, G).transpose(0, 2, 1) << bitpos).astype(np.uint8)
    return out.reshape(-1)


def split_a6(q):
    """q = 8 qh + ql with qh = floor(q / 8), ql = q - 8 qh (the A6 planes)."""
    q = np.asarray(q, dtype=np.int64)
    qh = np.floor_divide(q, 8)
    return qh, q - 8 * qh
