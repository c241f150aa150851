"""Per-token mean and centering, absmax integer codes, INT4 packing, MXFP4 codec.

Parity pins: tests/test_oracle_quant.py.

Sources:
  CentriQ Sec. 3 "Preliminaries", Eq. 1: symmetric b-bit per-token activation
  quantizer Q_a(x_t) = alpha_t clip(round(x_t / alpha_t), -(2^{b-1}-1),
  2^{b-1}-1) with alpha_t = r_t / (2^{b-1}-1) and r_t the largest coordinate
  magnitude of the token.
  CentriQ Sec. 4.2 "Activation path", Eq. 4: the token is centered over its n
  native channels, x^c = x - mean(x) 1; the mean is restored as a rank-1 term.
  CentriQ Sec. 4.2 "Activation path", "Scale and grid", and App. B.3
  (Table 3): the percentile scale.  The token's spread is the empirical
  rho-quantile of the rotated magnitudes divided by the half-normal quantile
  Phi^-1((1 + rho) / 2); the range is gamma* times that spread, with
  rho = 0.9995 and gamma* = 2.5591 fixed for all layers, and Eq. 1 then
  clips codes beyond the range.
  FLUX.1-schnell-OrbitQuant-W4A4 model card, "Quantization": activation
  normalization epsilon 1e-10; packed INT4 module tensors ("Artifact Files").
  WUSH review, "Core claim" and Fig. 2 caption: RTN AbsMax block quantizers,
  MXFP4 with group size 32; the review's reference list cites the OCP
  Microscaling (MX) v1.0 specification, which defines MXFP4 as E2M1 elements
  sharing one E8M0 power-of-two scale per 32.

Readings where the pages are silent:
  * round() is round-half-to-even;
  * x / alpha is evaluated as RN32(x * RN32(qmax / a)), one division per token;
  * an all-zero token uses max(a, eps32) with eps32 = RN32(1e-10), so every
    code is 0 and the scale is eps32 / qmax;
  * the mean is m = RN32(RN64(S) / d) with S the exact coordinate sum;
  * percentile scale: the empirical rho-quantile interpolates linearly
    between the order statistics k = floor(rho (n - 1)) and k + 1 of the
    magnitudes (ascending, 0-based), in float64; the range is
    r = RN32((q * gamma*) / z) with z = Phi^-1(1 - 0.00025) (the upper tail
    (1 - rho) / 2 taken as the decimal 0.00025), evaluated in that order in
    float64; gamma* = 2.5591 (Table 3; the text rounds it to 2.56); the
    scale and codes then follow the absmax rule with r in place of a;
  * INT4 packing: element 2i in bits 3..0, element 2i+1 in bits 7..4, 4-bit
    two's complement;
  * E8M0 shared exponent e = clamp(floor(log2 a) - 2, -127, 127) (the MX
    rule with emax(E2M1) = 2; a = 0 gives e = -127), elements rounded to the
    nearest E2M1 value, ties to the even code, magnitudes beyond 6 saturate,
    the sign bit copies the input's sign bit.
"""
from __future__ import annotations

import math

import numpy as np

EPS32 = np.float32(1e-10)

# OCP MX v1.0 E2M1 magnitudes, indexed by the 3-bit code (e1 e0 m)
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def qmax_for_bits(b: int) -> int:
    """2^{b-1} - 1 (Eq. 1): 127 for 8 bits, 31 for 6, 7 for 4."""
    return (1 << (b - 1)) - 1


# ---------------------------------------------------------------- centering --

def token_mean(x32: np.ndarray) -> np.ndarray:
    """m_t = RN32(RN64(sum_j x_tj) / d), sum taken exactly (math.fsum)."""
    x = np.asarray(x32, dtype=np.float64)
    d = x.shape[-1]
    s = np.array([math.fsum(row) for row in x.reshape(-1, d)], dtype=np.float64)
    return (s / float(d)).astype(np.float32).reshape(x.shape[:-1])


def fp64_sum_is_exact(x32: np.ndarray) -> bool:
    """Sufficient condition for every float64 partial sum of a row of
    bfloat16 values to be exact (so any summation order gives the exact sum):
    all values are multiples of 2^(emin-7) and every partial sum is below
    d * 2^(emax+1), which must fit in 53 bits."""
    x = np.abs(np.asarray(x32, dtype=np.float64))
    nz = x[x > 0]
    if nz.size == 0:
        return True
    emax = int(np.floor(np.log2(nz.max())))
    emin = int(np.floor(np.log2(nz.min())))
    d = x.shape[-1]
    bits = (emax + 1 + int(math.ceil(math.log2(d)))) - (emin - 7)
    return bits <= 53


def center(x32: np.ndarray, m: np.ndarray) -> np.ndarray:
    """x^c = RN32(x - m) per coordinate."""
    return (np.asarray(x32, dtype=np.float32) - np.asarray(m, dtype=np.float32)[..., None]).astype(np.float32)


# ------------------------------------------------------- integer quantizers --

def absmax_scale(a: np.ndarray, qmax: int):
    """(alpha, inv) from the range a: alpha = RN32(max(a,eps)/qmax),
    inv = RN32(qmax/max(a,eps))."""
    ae = np.maximum(np.asarray(a, dtype=np.float32), EPS32)
    q = np.float32(qmax)
    return (ae / q).astype(np.float32), (q / ae).astype(np.float32)


def round_codes(v32: np.ndarray, inv: np.ndarray, qmax: int):
    """q = clip(RNE(RN32(v * inv)), -qmax, qmax), plus the boundary flags:
    an element is flagged when its scaled value lies within 1e-6 relative of
    a half-integer (where one float32 ulp elsewhere could flip the code)."""
    t = (np.asarray(v32, dtype=np.float32) * inv).astype(np.float32)
    q = np.clip(np.rint(t), -qmax, qmax).astype(np.int32)
    t64 = t.astype(np.float64)
    half = np.floor(t64) + 0.5
    flag = np.abs(t64 - half) <= 1e-6 * np.abs(t64)
    return q, flag


def quant_token_int(v32: np.ndarray, qmax: int):
    """Per-token (last axis) absmax quantizer of Eq. 1.

    Returns (codes int32, alpha float32 [rows], boundary flags)."""
    v32 = np.asarray(v32, dtype=np.float32)
    a = np.max(np.abs(v32), axis=-1)
    alpha, inv = absmax_scale(a, qmax)
    q, flag = round_codes(v32, inv[..., None], qmax)
    return q, alpha, flag


PCTL_RHO = 0.9995
PCTL_GAMMA = 2.5591
PCTL_TAIL = 0.00025  # (1 - rho) / 2


def std_normal_upper_quantile(tail: float) -> float:
    """x with Phi(-x) = tail, i.e. Phi^-1(1 - tail): bisection on
    erfc(x / sqrt 2) / 2 = tail (the upper tail keeps full float64 precision),
    run until the bracket cannot shrink."""
    lo, hi = 0.0, 40.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if 0.5 * math.erfc(mid / math.sqrt(2.0)) > tail:
            lo = mid
        else:
            hi = mid
    return hi


def pctl_range(v32: np.ndarray, rho: float = PCTL_RHO, gamma: float = PCTL_GAMMA) -> np.ndarray:
    """Percentile range per token (last axis): r = RN32((q * gamma) / z), q the
    linearly interpolated empirical rho-quantile of the magnitudes."""
    a = np.sort(np.abs(np.asarray(v32, dtype=np.float32)).astype(np.float64), axis=-1)
    n = a.shape[-1]
    h = rho * (n - 1)
    k = int(math.floor(h))
    f = h - k
    lo = a[..., k]
    hi = a[..., min(k + 1, n - 1)]
    q = lo + f * (hi - lo)
    z = std_normal_upper_quantile(PCTL_TAIL)
    return ((q * gamma) / z).astype(np.float32)


def quant_token_pctl(v32: np.ndarray, qmax: int):
    """Per-token quantizer of Eq. 1 with the percentile range (codes beyond
    the range clip to +-qmax).  Returns (codes int32, alpha float32, flags)."""
    v32 = np.asarray(v32, dtype=np.float32)
    alpha, inv = absmax_scale(pctl_range(v32), qmax)
    q, flag = round_codes(v32, inv[..., None], qmax)
    return q, alpha, flag


def quant_groups_int(w32: np.ndarray, group: int, qmax: int = 7):
    """Symmetric absmax quantizer per (row, group of `group` consecutive
    input columns): the same rule as Eq. 1 with the range taken per group.

    Returns (codes int32 [N, K], scales float32 [N, K/group], flags)."""
    w32 = np.asarray(w32, dtype=np.float32)
    N, K = w32.shape
    g = w32.reshape(N, K // group, group)
    a = np.max(np.abs(g), axis=-1)
    s, inv = absmax_scale(a, qmax)
    q, flag = round_codes(g, inv[..., None], qmax)
    return q.reshape(N, K), s, flag.reshape(N, K)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two 4-bit two's-complement codes per byte, even element in the low nibble."""
    q = np.asarray(q, dtype=np.int64)
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int32)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# -------------------------------------------------------------------- MXFP4 --

def e8m0_exponent(a: np.ndarray) -> np.ndarray:
    """Shared exponent e = clamp(floor(log2 a) - 2, -127, 127); a = 0 -> -127."""
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)                  # a = m 2^ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1 - 2
    e = np.where(a == 0, -127, e)
    return np.clip(e, -127, 127)


def e2m1_encode(t: np.ndarray) -> np.ndarray:
    """Nearest E2M1 value (ties to the even code), saturating at 6; 4-bit
    code s e1 e0 m with the sign bit copied from the input."""
    t = np.asarray(t, dtype=np.float64)
    mag = np.minimum(np.abs(t), 6.0)
    dist = np.abs(mag[..., None] - E2M1_GRID)
    best = np.min(dist, axis=-1, keepdims=True)
    cand = dist == best
    # among equally near codes take the even one (lowest mantissa bit 0)
    idx = np.arange(8)
    even_pick = np.where(cand & (idx % 2 == 0), idx, 99).min(axis=-1)
    any_pick = np.where(cand, idx, 99).min(axis=-1)
    code = np.where(cand.sum(axis=-1) > 1, even_pick, any_pick)
    sign = np.signbit(t).astype(np.int64)
    return (code | (sign << 3)).astype(np.uint8)


def e2m1_decode(c: np.ndarray) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64)
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def quant_mx(v32: np.ndarray):
    """MXFP4 of every consecutive 32-block of the last axis.

    Returns (codes uint8 [.., d] one code per element, scale bytes uint8
    [.., d/32] = e + 127, element flags, block flags)."""
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    d = v.shape[-1]
    vb = v.reshape(v.shape[:-1] + (d // 32, 32))
    a = np.max(np.abs(vb), axis=-1)
    e = e8m0_exponent(a)
    t = np.ldexp(vb, -e[..., None])
    codes = e2m1_encode(t).reshape(v.shape)
    mag = np.abs(t)
    eflag = np.any(np.abs(mag[..., None] - E2M1_MIDPOINTS) <= 1e-6 * np.maximum(mag[..., None], 1e-300), axis=-1)
    with np.errstate(divide="ignore"):
        p2 = np.exp2(np.round(np.log2(np.where(a > 0, a, 1.0))))
    bflag = (a > 0) & (np.abs(a - p2) <= 1e-6 * a)
    return codes, (e + 127).astype(np.uint8), eflag.reshape(v.shape), bflag


def mx_dequant(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """Real value of each MXFP4 element: E2M1 value times 2^(X - 127)."""
    vals = e2m1_decode(codes)
    d = vals.shape[-1]
    vb = vals.reshape(vals.shape[:-1] + (d // 32, 32))
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    return np.ldexp(vb, e[..., None]).reshape(vals.shape)


def pack_nibbles(c: np.ndarray) -> np.ndarray:
    """Unsigned 4-bit fields two per byte, even element in the low nibble."""
    c = np.asarray(c, dtype=np.int64)
    return ((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = (b >> 4) & 0xF
    return out
