"""Lloyd-Max activation codebook for rotated tokens, its nearest-centroid
quantizer, and the dequantizing product it feeds.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Parity pins: tests/test_oracle_lloyd_max.py.

Sources:
  OrbitQuant PR #25, "Default changes": Lloyd-Max activation codes are the
  method's own activation quantizer (the default below 8 bits); codebooks are
  built per layer width d (the table build is timed per width up to
  d = 30720, and the newer builder is a Newton solver).
  CentriQ, Sec. 2 "Related work", paragraph on calibration-free quantizers:
  OrbitQuant's Lloyd-Max codebook is derived from the post-rotation marginal
  (following Zandieh et al.), with no calibration data.
  FLUX.1-schnell-OrbitQuant-W4A4 model card, "Quantization": codebook
  lloyd_max, activation normalization epsilon 1e-10, "Artifact Files": the
  Lloyd-Max codebooks are stored with the model.

Readings where the pages are silent:
  * the post-rotation marginal is that of one coordinate of a point drawn
    uniformly from the unit sphere S^{d-1}: density proportional to
    (1 - t^2)^((d - 3) / 2) on [-1, 1];
  * tokens are normalized by their root-mean-square rho = ||v|| / sqrt(d),
    so the codebook is built for u = sqrt(d) t (unit variance) and the
    dequantized value is rho * c[q];
  * the codebook has L = 2^b levels and minimizes E[(U - Q(U))^2]: every
    level is the mean of U over its cell and every cell boundary is the
    midpoint of its two levels (Lloyd's two conditions); the marginal is even,
    so the levels are symmetric and, for even L, 0 is a boundary;
  * stored codebook: levels rounded to float16 (RNE), ascending; the decision
    thresholds are the exact midpoints of adjacent stored levels (exact in
    float32), so the quantizer is the nearest stored level;
  * rho = RN32(sqrt(RN64(S) / d)) with S the exact sum of squares of the
    float32 rotated values, evaluated in float64; rho is floored at
    RN32(1e-10); u = RN32(v * RN32(1 / rho));
  * code = number of thresholds strictly below u (a tie goes to the lower
    level); codes are the level indices 0 .. L-1;
  * the product dequantizes both operands to float16: weights as
    RN16(s * q) from their INT4 codes q and group scales s, activations as
    their stored levels; float16 x float16 products are exact, and the
    reference result is RN32(float64(rho_t * sum_k c[q_tk] W16[o, k]
    + m_t w1[o] + b[o])).
"""
from __future__ import annotations

import math

import numpy as np
from scipy import optimize, special

EPS32 = np.float32(1e-10)


# ---------------------------------------------------------------- the marginal
def _shape(d: int) -> float:
    if d < 3:
        raise ValueError("the sphere marginal needs d >= 3")
    return (d - 1) / 2.0


def upper_tail(u, d: int) -> np.ndarray:
    """P(U > u) for u >= 0, U = sqrt(d) T, T one coordinate of a uniform point
    on S^{d-1}.  T^2 ~ Beta(1/2, (d-1)/2), so P(|T| > t) = 1 - I_{t^2}."""
    u = np.asarray(u, dtype=np.float64)
    t2 = np.minimum((u / math.sqrt(d)) ** 2, 1.0)
    return 0.5 * special.betaincc(0.5, _shape(d), t2)


def _cell_mass(a, b, d):
    """P(a < U <= b) for 0 <= a < b, from whichever tail form is small."""
    n = _shape(d)
    ta = np.minimum((a / math.sqrt(d)) ** 2, 1.0)
    tb = np.minimum((b / math.sqrt(d)) ** 2, 1.0)
    lo = 0.5 * (special.betainc(0.5, n, tb) - special.betainc(0.5, n, ta))
    hi = 0.5 * (special.betaincc(0.5, n, ta) - special.betaincc(0.5, n, tb))
    return np.where(special.betainc(0.5, n, ta) < 0.5, lo, hi)


def _cell_moment(a, b, d):
    """int_a^b u g(u) du for 0 <= a < b.  With t = u / sqrt(d),
    d/dt[-(1 - t^2)^((d-1)/2)] = (d - 1) t (1 - t^2)^((d-3)/2), so the moment
    is sqrt(d) (E(a) - E(b)) / ((d - 1) B(1/2, (d-1)/2)) with
    E(u) = (1 - t^2)^((d-1)/2), differenced without cancellation."""
    n = _shape(d)
    sd = math.sqrt(d)
    norm = sd / ((d - 1) * special.beta(0.5, n))
    ta = np.minimum((np.asarray(a, float) / sd) ** 2, 1.0)
    tb = np.minimum((np.asarray(b, float) / sd) ** 2, 1.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        xa = n * np.log1p(-ta)
        xb = n * np.log1p(-tb)
        both = np.exp(xb) * np.expm1(xa - xb)
    out = np.where(np.isfinite(xb), both, np.exp(xa))
    return norm * out


# ---------------------------------------------------------------- the codebook
def _half_centroids(p, d):
    """Centroids of the cells [p_i, p_{i+1}] of the positive half, with
    p_0 = 0 and the last edge at sqrt(d)."""
    edges = np.concatenate([[0.0], p, [math.sqrt(d)]])
    return _cell_moment(edges[:-1], edges[1:], d) / _cell_mass(edges[:-1], edges[1:], d)


def _residual(p, d):
    """Each interior boundary minus the midpoint of its two centroids."""
    c = _half_centroids(p, d)
    return p - 0.5 * (c[:-1] + c[1:])


def lloyd_max_levels(d: int, bits: int, lloyd_iters: int = 40):
    """Float64 Lloyd-Max levels (ascending, 2^bits of them) for the unit-variance
    sphere marginal of width d, with the fixed-point residual reached.

    The positive half is solved (the marginal is even): start from boundaries
    at equal-probability quantiles, take a few Lloyd steps (centroids, then
    midpoints), then solve residual(p) = 0 with a library root finder."""
    L = 1 << bits
    h = L // 2
    n = _shape(d)
    if h == 1:
        c = _half_centroids(np.zeros(0), d)
        return np.concatenate([-c[::-1], c]), 0.0
    # P(U > p) = (h - i) / L  <=>  I_{t^2}(1/2, n) = 1 - 2 (h - i) / L
    probs = 1.0 - 2.0 * (h - np.arange(1, h)) / L
    p = math.sqrt(d) * np.sqrt(special.betaincinv(0.5, n, probs))
    for _ in range(lloyd_iters):
        c = _half_centroids(p, d)
        p = 0.5 * (c[:-1] + c[1:])
    sol = optimize.root(_residual, p, args=(d,), method="hybr", tol=1e-15)
    p = sol.x
    res = float(np.abs(_residual(p, d)).max())
    c = _half_centroids(p, d)
    return np.concatenate([-c[::-1], c]), res


def mse(levels, d: int) -> float:
    """E[(U - Q(U))^2] of the nearest-level quantizer, by the cell integrals
    (E[U^2] = 1, so MSE = 1 - sum_i c_i (2 M_i - c_i P_i) with M_i the cell's
    first moment and P_i its mass, summed over both halves)."""
    c = np.asarray(levels, float)
    pos = c[c > 0]
    edges = np.concatenate([[0.0], 0.5 * (pos[:-1] + pos[1:]), [math.sqrt(d)]])
    P = _cell_mass(edges[:-1], edges[1:], d)
    M = _cell_moment(edges[:-1], edges[1:], d)
    return float(1.0 - 2.0 * np.sum(pos * (2 * M - pos * P)))


def codebook_tables(d: int, bits: int):
    """(levels float16 [L], thresholds float32 [L - 1]) as the kernels consume
    them: RNE float16 levels, thresholds the exact float32 midpoints."""
    lv, _ = lloyd_max_levels(d, bits)
    c16 = lv.astype(np.float16)
    c32 = c16.astype(np.float32)
    thr = (c32[:-1] + c32[1:]) * np.float32(0.5)
    assert np.array_equal(thr.astype(np.float64), 0.5 * (c16[:-1].astype(np.float64) + c16[1:].astype(np.float64)))
    return c16, thr


# ---------------------------------------------------------------- quantizer
def rms_f64(v32: np.ndarray) -> np.ndarray:
    """sqrt(RN64(S_t) / d) in float64, S_t the exact sum of squares of the
    float32 rotated coordinates (each square is exact in float64)."""
    v32 = np.asarray(v32, dtype=np.float32)
    d = v32.shape[1]
    out = np.empty(v32.shape[0], dtype=np.float64)
    for t in range(v32.shape[0]):
        S = math.fsum(float(x) * float(x) for x in v32[t])
        out[t] = math.sqrt(S / d)
    return out


def rms_scale(v32: np.ndarray) -> np.ndarray:
    """rho_t = max(RN32(sqrt(RN64(S_t) / d)), RN32(1e-10))."""
    return np.maximum(rms_f64(v32).astype(np.float32), EPS32)


def boundary_flags(v32: np.ndarray, rho: np.ndarray, thr32: np.ndarray) -> np.ndarray:
    """Elements whose u = RN32(v RN32(1 / rho)) lies within 1e-6 (relative)
    of a decision threshold (the rounding-boundary exemption)."""
    v32 = np.asarray(v32, dtype=np.float32)
    inv = (np.float32(1.0) / np.asarray(rho, np.float32)).astype(np.float32)
    u = (v32 * inv[:, None]).astype(np.float32).astype(np.float64)
    t = np.asarray(thr32, np.float64)
    i = np.clip(np.searchsorted(t, u), 1, t.size - 1) if t.size > 1 else np.zeros(u.shape, np.int64)
    near = np.minimum(np.abs(u - t[i]), np.abs(u - t[np.maximum(i - 1, 0)]))
    return near <= 1e-6 * np.abs(u)


def quant_token_lm(v32: np.ndarray, thr32: np.ndarray):
    """Lloyd-Max codes (uint8 level indices) and rho per token."""
    v32 = np.asarray(v32, dtype=np.float32)
    rho = rms_scale(v32)
    inv = (np.float32(1.0) / rho).astype(np.float32)
    u = (v32 * inv[:, None]).astype(np.float32)
    q = np.searchsorted(np.asarray(thr32, np.float32), u, side="left")
    return q.astype(np.uint8), rho


def weights_f16(qw: np.ndarray, w_scale: np.ndarray, group: int) -> np.ndarray:
    """W16[o, k] = RN16(s[o, k // group] * q[o, k]) (the product is exact in
    float64, then rounded once)."""
    s = np.repeat(np.asarray(w_scale, np.float64), group, axis=1)
    return (s * np.asarray(qw, np.float64)).astype(np.float16)


def linear_lm(codes, rho, c16, w16, mean=None, w1=None, bias=None):
    """Reference output RN32(float64(rho_t sum_k c16[q] W16 + m w1 + b)) and the
    magnitude sum S of its terms (for the output tolerance)."""
    a = np.asarray(c16, np.float64)[np.asarray(codes, np.int64)]
    W = np.asarray(w16, np.float64)
    acc = a @ W.T
    accS = np.abs(a) @ np.abs(W).T
    r = np.asarray(rho, np.float64)[:, None]
    y = r * acc
    S = r * accS
    if mean is not None:
        y = y + np.asarray(mean, np.float64)[:, None] * np.asarray(w1, np.float64)[None, :]
        S = S + np.abs(np.asarray(mean, np.float64)[:, None] * np.asarray(w1, np.float64)[None, :])
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
        S = S + np.abs(np.asarray(bias, np.float64))[None, :]
    return y.astype(np.float32), S
