"""NumPy writer of the tiled FP6 operand layout, from its definition in
include/oq.h (a data layout, no arithmetic of the method): rows padded to 32,
K a multiple of 64, tile (r/32, kg = k/64) of 1536 bytes at
((r/32) * (K/64) + kg) * 1536.  The 32 codes of row r and k-half h form a
192-bit string with code j in bits [6j, 6j+6); with l = 32 h + r % 32, its
bytes 0..15 sit at tile + 16 l and bytes 16..23 at tile + 1024 + 8 l.
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


def _strings(codes: np.ndarray) -> np.ndarray:
    """int codes [Rp, K] -> the 24-byte strings [Rp, K/64, 2, 24] of (row, kg, half)."""
    Rp, K = codes.shape
    G = K // 64
    f = e2m3(codes).reshape(Rp, G, 2, 32)
    out = np.zeros((Rp, G, 2, 24), dtype=np.uint8)
    for j in range(32):
        for b in range(6):
            pos = 6 * j + b
            bit = ((f[..., j] >> np.uint64(b)) & np.uint64(1)).astype(np.uint8)
            out[..., pos // 8] |= (bit << (pos % 8)).astype(np.uint8)
    return out


def tile(codes: np.ndarray) -> np.ndarray:
    """int codes [R, K] in [-7, 7] -> tiled bytes (R padded to 32)."""
    R, K = codes.shape
    assert K % 64 == 0
    Rp = (R + 31) // 32 * 32
    G = K // 64
    c = np.zeros((Rp, K), dtype=np.int64)
    c[:R] = codes
    st = _strings(c).reshape(Rp // 32, 32, G, 2, 24).transpose(0, 2, 3, 1, 4)  # [rb, kg, h, r, 24]
    out = np.zeros((Rp // 32, G, 1536), dtype=np.uint8)
    out[:, :, :1024] = st[..., :16].reshape(Rp // 32, G, 1024)   # l = 32 h + r, 16 bytes each
    out[:, :, 1024:] = st[..., 16:].reshape(Rp // 32, G, 512)    # 8 bytes each
    return out.reshape(-1)


def row_mask(R: int, K: int) -> np.ndarray:
    """Boolean mask over the tiled bytes of R rows (padded to 32): True where the
    byte belongs to a row < R (padding rows are never written by the kernels)."""
    Rp = (R + 31) // 32 * 32
    G = K // 64
    rows = np.arange(Rp).reshape(Rp // 32, 32)
    live = rows < R                                              # [rb, r]
    lane = np.concatenate([live, live], axis=1)                  # l = 32 h + r
    m = np.zeros((Rp // 32, G, 1536), dtype=bool)
    m[:, :, :1024] = np.repeat(lane, 16, axis=1)[:, None, :]
    m[:, :, 1024:] = np.repeat(lane, 8, axis=1)[:, None, :]
    return m.reshape(-1)


def split_a6(q):
    """q = 8 qh + ql with qh = floor(q / 8), ql = q - 8 qh (the A6 planes)."""
    q = np.asarray(q, dtype=np.int64)
    qh = np.floor_divide(q, 8)
    return qh, q - 8 * qh


def tile_mx(codes: np.ndarray, e8m0: np.ndarray):
    """Row-major MXFP4 codes [R, K/2] (two E2M1 codes per byte) and E8M0 bytes
    [R, K/32] -> (tiled codes, tiled scale words) as defined in include/oq.h:
    tile (r/32, kg) of 1024 bytes holds at 16 (32 h + r % 32) the 16 code bytes
    of row r, k-half h; the scale word of (k-slice s, row r) sits at byte
    (s * Rp + r) * 4 with the E8M0 bytes of blocks 4s..4s+3.  Padding rows get
    zero codes and scale 127."""
    R, Kh = codes.shape
    K = 2 * Kh
    assert K % 128 == 0 and e8m0.shape == (R, K // 32)
    Rp = (R + 31) // 32 * 32
    G = K // 64
    c = np.zeros((Rp, Kh), dtype=np.uint8)
    c[:R] = codes
    e = np.full((Rp, K // 32), 127, dtype=np.uint8)
    e[:R] = e8m0
    t = c.reshape(Rp // 32, 32, G, 2, 16).transpose(0, 2, 3, 1, 4)   # [rb, kg, h, r, 16]
    tiled = np.ascontiguousarray(t).reshape(-1)
    sc = e.reshape(Rp, K // 128, 4).transpose(1, 0, 2)               # [s, r, 4]
    return tiled, np.ascontiguousarray(sc).reshape(-1)


def row_mask_mx(R: int, K: int) -> np.ndarray:
    """Boolean mask over the tiled MXFP4 code bytes of R rows: True for rows < R."""
    Rp = (R + 31) // 32 * 32
    G = K // 64
    live = (np.arange(Rp) < R).reshape(Rp // 32, 1, 1, 32, 1)
    return np.broadcast_to(live, (Rp // 32, G, 2, 32, 16)).reshape(-1)



# ---------------------------------------------------------------- float16 tiles
# Tiled float16 operand layout (include/oq.h, oq_tiled_f16_bytes): rows padded
# to 32, chunk (r / 32, k / 16) of 512 float16 at ((r / 32) * (K / 16) + k / 16)
# * 512; lane l = 32 * ((k % 16) // 8) + r % 32 holds k % 8 = 0..7 at 8 l.
def tile_f16(vals: np.ndarray) -> np.ndarray:
    """uint16 [R, K] -> tiled uint16 (R padded to 32 with zeros)."""
    R, K = vals.shape
    assert K % 16 == 0
    Rp = (R + 31) // 32 * 32
    v = np.zeros((Rp, K), dtype=np.uint16)
    v[:R] = vals
    return v.reshape(Rp // 32, 32, K // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1).copy()


def untile_f16(buf: np.ndarray, R: int, K: int) -> np.ndarray:
    """tiled uint16 -> [R padded to 32, K]."""
    Rp = (R + 31) // 32 * 32
    b = np.asarray(buf).view(np.uint16)[: Rp * K]
    return b.reshape(Rp // 32, K // 16, 2, 32, 8).transpose(0, 3, 1, 2, 4).reshape(Rp, K)


# E2M3 magnitudes from the format definition: bits e (2) m (3), e = 0 gives
# m / 8, else 2^(e - 1) (1 + m / 8); used for values other than integers
E2M3_MAGNITUDES = np.array([(m / 8.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 8.0)
                            for e in range(4) for m in range(8)])


def e2m3_bits(x) -> np.ndarray:
    """E2M3 bit patterns of values that the format holds exactly."""
    x = np.asarray(x, dtype=np.float64)
    idx = np.array([np.flatnonzero(E2M3_MAGNITUDES == abs(v))[0] for v in x.ravel()], dtype=np.uint64)
    sign = np.where(np.signbit(x.ravel()) & (x.ravel() != 0), np.uint64(0x20), np.uint64(0))
    return (idx | sign).reshape(x.shape)


def tile_values(vals: np.ndarray) -> np.ndarray:
    """E2M3-exact values [R, K] -> tiled bytes (the layout of tile())."""
    R, K = vals.shape
    Rp = (R + 31) // 32 * 32
    G = K // 64
    f = np.zeros((Rp, K), dtype=np.uint64)
    f[:R] = e2m3_bits(vals)
    f = f.reshape(Rp, G, 2, 32)
    st = np.zeros((Rp, G, 2, 24), dtype=np.uint8)
    for j in range(32):
        for b in range(6):
            pos = 6 * j + b
            bit = ((f[..., j] >> np.uint64(b)) & np.uint64(1)).astype(np.uint8)
            st[..., pos // 8] |= (bit << (pos % 8)).astype(np.uint8)
    st = st.reshape(Rp // 32, 32, G, 2, 24).transpose(0, 2, 3, 1, 4)
    out = np.zeros((Rp // 32, G, 1536), dtype=np.uint8)
    out[:, :, :1024] = st[..., :16].reshape(Rp // 32, G, 1024)
    out[:, :, 1024:] = st[..., 16:].reshape(Rp // 32, G, 512)
    return out.reshape(-1)


# ------------------------------------------------------------- layout readers
def untile(buf: np.ndarray, R: int, K: int) -> np.ndarray:
    """Tiled FP6 bytes (one plane) -> int codes [R, K]: the inverse of tile(),
    decoding each 6-bit field as E2M3 (sign bit 5, exponent bits 4..3 with
    bias 1, mantissa bits 2..0); every field must hold an integer value."""
    Rp = (R + 31) // 32 * 32
    G = K // 64
    b = np.asarray(buf).view(np.uint8)[: Rp // 32 * G * 1536].reshape(Rp // 32, G, 1536)
    st = np.zeros((Rp // 32, G, 2, 32, 24), dtype=np.uint8)            # [rb, kg, h, r, 24]
    st[..., :16] = b[:, :, :1024].reshape(Rp // 32, G, 2, 32, 16)
    st[..., 16:] = b[:, :, 1024:].reshape(Rp // 32, G, 2, 32, 8)
    bits = np.unpackbits(st, axis=-1, bitorder="little")                # [.., 192]
    fields = bits.reshape(st.shape[:-1] + (32, 6)).astype(np.int64)
    f = np.zeros(fields.shape[:-1], dtype=np.int64)
    for k in range(6):
        f |= fields[..., k] << k
    mag = E2M3_MAGNITUDES[f & 0x1F]
    val = np.where(f & 0x20, -mag, mag)
    assert np.all(val == np.rint(val)), "non-integer FP6 field"
    codes = val.astype(np.int64).transpose(0, 3, 1, 2, 4).reshape(Rp, K)  # [rb, r, kg, h, j]
    return codes[:R]


def untile_mx(buf: np.ndarray, sbuf: np.ndarray, R: int, K: int):
    """Tiled MXFP4 codes and scale words -> (row-major code bytes [R, K/2],
    E8M0 bytes [R, K/32]): the inverse of tile_mx()."""
    Rp = (R + 31) // 32 * 32
    G = K // 64
    t = np.asarray(buf).view(np.uint8)[: Rp * K // 2].reshape(Rp // 32, G, 2, 32, 16)
    codes = t.transpose(0, 3, 1, 2, 4).reshape(Rp, K // 2)
    sc = np.asarray(sbuf).view(np.uint8)[: Rp * K // 32].reshape(K // 128, Rp, 4)
    e8m0 = sc.transpose(1, 0, 2).reshape(Rp, K // 32)
    return codes[:R], e8m0[:R]
