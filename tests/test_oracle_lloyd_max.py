"""Pins of the Lloyd-Max oracle (oracle/lloyd_max.py) against facts outside it.

* d = 3: one coordinate of a uniform point on S^2 is uniform on [-1, 1]
  (Archimedes' hat-box theorem), so the optimal L-level quantizer is the
  uniform one: levels sqrt(3) ((2i + 1) / L - 1), MSE 1 / L^2.
* d large: sqrt(d) T tends to a standard normal, and the levels approach the
  Gaussian Lloyd-Max quantizers tabulated by J. Max, "Quantizing for minimum
  distortion", IRE Trans. Inform. Theory, 1960 (4-decimal table values).
* The closed-form cell mass and moment against numerical quadrature of the
  density, and Monte Carlo samples of the sphere against the cell masses and
  levels (this pins the density's exponent).
* The threshold quantizer against a brute-force nearest-level search; the
  RMS scale against constant rows and power-of-two scaling; the product
  against a plain loop.
"""
import math

import numpy as np
import pytest
from scipy import integrate, special

from oracle import lloyd_max as LM

# J. Max (1960), Gaussian, minimum-MSE: positive output levels and MSE
MAX_TABLE = {
    1: ([0.7979], 0.3634),
    2: ([0.4528, 1.510], 0.1175),
    3: ([0.2451, 0.7560, 1.344, 2.152], 0.03454),
    4: ([0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733], 0.009497),
}


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_uniform_marginal_at_d3(bits):
    L = 1 << bits
    lv, res = LM.lloyd_max_levels(3, bits)
    want = math.sqrt(3) * ((2 * np.arange(L) + 1) / L - 1)
    assert res < 1e-12
    np.testing.assert_allclose(lv, want, rtol=0, atol=1e-12)
    assert abs(LM.mse(lv, 3) - 1.0 / L ** 2) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_limit_matches_max_table(bits):
    levels, m = MAX_TABLE[bits]
    lv, res = LM.lloyd_max_levels(30720, bits)
    assert res < 1e-12
    pos = lv[lv > 0]
    np.testing.assert_allclose(pos, levels, rtol=0, atol=2e-3)
    assert abs(LM.mse(lv, 30720) - m) < 0.01 * m


@pytest.mark.parametrize("d", [4, 5, 17, 100])
def test_cell_integrals_against_quadrature(d):
    B = special.beta(0.5, (d - 1) / 2)
    sd = math.sqrt(d)

    def g(u):  # density of U = sqrt(d) T
        return (1 - (u / sd) ** 2) ** ((d - 3) / 2) / (B * sd)

    for a, b in [(0.0, 0.3), (0.3, 1.1), (1.1, 0.999 * sd), (0.0, sd)]:
        P = integrate.quad(g, a, b, epsabs=1e-14, epsrel=1e-12)[0]
        M = integrate.quad(lambda u: u * g(u), a, b, epsabs=1e-14, epsrel=1e-12)[0]
        assert abs(LM._cell_mass(np.array([a]), np.array([b]), d)[0] - P) < 1e-10
        assert abs(LM._cell_moment(np.array([a]), np.array([b]), d)[0] - M) < 1e-10
    # whole positive half: mass 1/2, and the variance of U is 1
    assert abs(LM._cell_mass(np.array([0.0]), np.array([sd]), d)[0] - 0.5) < 1e-13
    var = 2 * integrate.quad(lambda u: u * u * g(u), 0, sd, epsabs=1e-14, epsrel=1e-12)[0]
    assert abs(var - 1.0) < 1e-10


def test_monte_carlo_sphere_coordinates():
    d, bits = 24, 3
    lv, _ = LM.lloyd_max_levels(d, bits)
    rng = np.random.default_rng(5)
    g = rng.standard_normal((200_000, d))
    u = math.sqrt(d) * (g[:, :2] / np.linalg.norm(g, axis=1, keepdims=True)).ravel()
    thr = 0.5 * (lv[:-1] + lv[1:])
    cell = np.searchsorted(thr, u)
    n = u.size
    edges = np.concatenate([[-math.sqrt(d)], thr, [math.sqrt(d)]])
    for i in range(lv.size):
        a, b = edges[i], edges[i + 1]
        if a >= 0:
            P = LM._cell_mass(np.array([a]), np.array([b]), d)[0]
        else:  # mirror image of a positive cell
            P = LM._cell_mass(np.array([-b]), np.array([-a]), d)[0]
        sel = u[cell == i]
        assert abs(sel.size / n - P) < 5 * math.sqrt(P * (1 - P) / n) + 1e-4
        # the level is the cell mean (Lloyd's centroid condition)
        assert abs(sel.mean() - lv[i]) < 5 * sel.std() / math.sqrt(sel.size) + 1e-4


@pytest.mark.parametrize("d,bits", [(32, 4), (3072, 4), (4096, 8), (128, 8)])
def test_lloyd_conditions_and_tables(d, bits):
    lv, res = LM.lloyd_max_levels(d, bits)
    assert res < 1e-11
    assert np.all(np.diff(lv) > 0)
    np.testing.assert_array_equal(lv, -lv[::-1])
    c16, thr = LM.codebook_tables(d, bits)
    assert c16.dtype == np.float16 and thr.dtype == np.float32
    assert c16.size == 1 << bits and thr.size == (1 << bits) - 1
    np.testing.assert_array_equal(c16, -c16[::-1])
    assert thr[(1 << bits) // 2 - 1] == 0.0
    # a perturbed codebook has a larger MSE (the levels are a minimum)
    m0 = LM.mse(lv, d)
    for i in (0, lv.size // 2, lv.size - 1):
        for eps in (1e-3, -1e-3):
            lp = lv.copy()
            lp[i] += eps
            lp[lv.size - 1 - i] -= eps  # keep it symmetric
            if np.all(np.diff(lp) > 0):
                assert LM.mse(lp, d) > m0


def _brute_nearest(u, c16):
    c = c16.astype(np.float64)
    out = np.empty(u.shape, np.uint8)
    for idx, x in np.ndenumerate(u):
        dist = np.abs(float(x) - c)
        out[idx] = int(np.flatnonzero(dist == dist.min())[0])  # ties: lower index
    return out


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_is_nearest_stored_level(bits):
    d = 256
    c16, thr = LM.codebook_tables(d, bits)
    rng = np.random.default_rng(bits)
    v = (rng.standard_normal((6, d)) * rng.uniform(0.1, 8, (6, 1))).astype(np.float32)
    v[0, :8] = 0.0
    q, rho = LM.quant_token_lm(v, thr)
    inv = (np.float32(1) / rho).astype(np.float32)
    u = (v * inv[:, None]).astype(np.float32)
    np.testing.assert_array_equal(q, _brute_nearest(u, c16))
    # exact ties on a threshold resolve to the lower level
    uu = np.concatenate([thr, c16.astype(np.float32)]).astype(np.float32)
    got = np.searchsorted(thr, uu, side="left")
    np.testing.assert_array_equal(got, _brute_nearest(uu, c16))


def test_rms_scale_closed_forms():
    d = 96
    v = np.full((3, d), 0.0, np.float32)
    v[0] = 3.0
    v[1, ::2], v[1, 1::2] = 1.5, -1.5
    rho = LM.rms_scale(v)
    assert rho[0] == np.float32(3.0) and rho[1] == np.float32(1.5)
    assert rho[2] == LM.EPS32
    c16, thr = LM.codebook_tables(d, 4)
    q, _ = LM.quant_token_lm(v, thr)
    # a zero row sits on the middle threshold (0): the lower central level
    assert np.all(q[2] == 7)
    # every element of a constant row has u = 1: the level nearest 1
    assert np.all(q[0] == _brute_nearest(np.array([1.0], np.float32), c16)[0])
    rng = np.random.default_rng(1)
    w = rng.standard_normal((4, d)).astype(np.float32)
    for k in (-20, 7):
        qs, rs = LM.quant_token_lm(np.ldexp(w, k).astype(np.float32), thr)
        q0, r0 = LM.quant_token_lm(w, thr)
        np.testing.assert_array_equal(qs, q0)
        np.testing.assert_array_equal(rs, np.ldexp(r0, k).astype(np.float32))


def test_weights_f16_rounding():
    q = np.array([[1, -7, 3, 0]], np.int64)
    s = np.array([[np.float32(0.1)]], np.float32)
    w = LM.weights_f16(q, s, 4)
    for j in range(4):
        exact = float(np.float32(0.1)) * int(q[0, j])
        assert w[0, j] == np.float16(exact)
        # RN16: no float16 is closer
        f = float(w[0, j])
        up = float(np.nextafter(w[0, j], np.float16(np.inf)))
        dn = float(np.nextafter(w[0, j], np.float16(-np.inf)))
        assert abs(f - exact) <= abs(up - exact) and abs(f - exact) <= abs(dn - exact)


def test_linear_lm_against_loop():
    rng = np.random.default_rng(3)
    M, K, N, g = 3, 64, 5, 32
    c16, thr = LM.codebook_tables(K, 4)
    codes = rng.integers(0, 16, (M, K)).astype(np.uint8)
    rho = rng.uniform(0.5, 2, M).astype(np.float32)
    qw = rng.integers(-7, 8, (N, K))
    sw = rng.uniform(0.001, 0.01, (N, K // g)).astype(np.float32)
    w16 = LM.weights_f16(qw, sw, g)
    mean = rng.standard_normal(M).astype(np.float32)
    w1 = rng.standard_normal(N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    y, S = LM.linear_lm(codes, rho, c16, w16, mean, w1, b)
    for t in range(M):
        for o in range(N):
            acc = math.fsum(float(c16[codes[t, k]]) * float(w16[o, k]) for k in range(K))
            ref = float(rho[t]) * acc + float(mean[t]) * float(w1[o]) + float(b[o])
            assert abs(float(y[t, o]) - ref) <= 1e-6 * abs(ref) + 1e-12
            assert S[t, o] >= abs(ref) - 1e-9


def test_rms_scale_rounds_the_exact_sum_once_then_to_float32():
    # rho = RN32(sqrt(RN64(S) / d)) with S the exact sum of squares.  Tokens of
    # d = 64 built so that rho sits at or next to the float32 midpoint
    # 1 + 2^-24 between 1 and 1 + 2^-23 (all coordinates bfloat16 values):
    #   A: 60 ones, 2, 2^-9, 2^-9, c = 2^-21: S = 64 + 2^-17 + 2^-42 =
    #      64 (1 + 2^-24)^2 exactly, rho is the midpoint -> even -> 1;
    #   B: c = 2^-21 (1 + 2^-7): S exceeds A's by 2^-48 + 2^-56, less than
    #      half a float64 ulp at 64 (2^-47), so RN64(S) is A's S -> 1 (a sum
    #      carried in more precision would round up);
    #   C: c = 1.5 2^-21: S exceeds A's by 1.25 2^-42 -> 1 + 2^-23;
    #   D: c = 1.5 2^-22: S is 0.4375 2^-42 below A's -> 1.
    def tok(c):
        return np.array([1.0] * 60 + [2.0, 2.0 ** -9, 2.0 ** -9, c], dtype=np.float32)
    v = np.stack([tok(2.0 ** -21), tok(2.0 ** -21 * (1 + 2.0 ** -7)), tok(1.5 * 2.0 ** -21), tok(1.5 * 2.0 ** -22)])
    up = np.float32(1.0 + 2.0 ** -23)
    np.testing.assert_array_equal(LM.rms_scale(v), np.array([1.0, 1.0, up, 1.0], dtype=np.float32))
