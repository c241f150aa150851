"""Pins of the asymmetric-weight oracle (oracle/asym.py): hand-worked RTN
examples (tests/golden/asym_rtn.txt), the nearest-grid-point property by brute
force, the reconstruction bound, scale invariance, the constant group, the
stored-offset identity sigma (Q - z) = sigma (Q - 8) - C, and the product
against a plain loop over dequantized weights."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import asym as OA
from oracle import quant as OQ

GOLD = os.path.join(os.path.dirname(__file__), "golden", "asym_rtn.txt")


def _golden():
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        g, w, s, z, q = [p.strip() for p in line.split("|")]
        yield int(g), np.array(w.split(), np.float32), float(s), float(z), np.array(q.split(), np.int64)


@pytest.mark.parametrize("case", list(_golden()), ids=lambda c: f"g{c[0]}")
def test_golden_rtn(case):
    g, w, s, z, q = case
    Q, sig, zz, flags = OA.quant_groups_asym(w[None, :], g)
    assert sig[0, 0] == s and zz[0, 0] == z
    np.testing.assert_array_equal(Q[0], q)
    assert not flags.any()


def _rand_weights(seed, N=6, K=256):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)) * 0.02
    W[1] += 0.05          # a row offset: the shift matters
    W[2, :64] = np.abs(W[2, :64])  # a one-signed group
    W[3, 64:128] = 0.0125  # a constant group
    return W.astype(np.float32)


def test_codes_are_nearest_grid_points():
    W = _rand_weights(1)
    Q, sig, z, flags = OA.quant_groups_asym(W, 64)
    s = np.repeat(sig, 64, axis=1).astype(np.float64)
    zz = np.repeat(z, 64, axis=1).astype(np.float64)
    grid = s[..., None] * (np.arange(16)[None, None, :] - zz[..., None])
    best = np.argmin(np.abs(grid - W.astype(np.float64)[..., None]), axis=-1)
    ok = (best == Q) | flags
    assert ok.all(), np.argwhere(~ok)[:5]
    assert Q.min() >= 0 and Q.max() <= 15


def test_reconstruction_bound_and_range():
    W = _rand_weights(2)
    Q, sig, z, _ = OA.quant_groups_asym(W, 64)
    err = np.abs(OA.dequant(Q, sig, z, 64) - W.astype(np.float64))
    s = np.repeat(sig, 64, axis=1).astype(np.float64)
    zz = np.repeat(np.abs(z), 64, axis=1).astype(np.float64)
    # half a step, plus the bfloat16 rounding of the shift (relative 2^-9) and
    # of the scale (relative 2^-9 over at most 15 steps)
    bound = 0.5 * s + s * zz * 2.0 ** -8 + 15 * s * 2.0 ** -8 + 1e-12
    assert (err <= bound).all()
    # min-max: the group's extremes use codes at (or next to) the ends
    g = W.reshape(6, 4, 64)
    qg = Q.reshape(6, 4, 64)
    lo = np.take_along_axis(qg, np.argmin(g, axis=-1)[..., None], -1)
    hi = np.take_along_axis(qg, np.argmax(g, axis=-1)[..., None], -1)
    assert np.all(lo <= 1) and np.all((hi >= 14) | (g.max(-1) == g.min(-1))[..., None])


def test_constant_group_and_scale_invariance():
    W = _rand_weights(3)
    Q, sig, z, _ = OA.quant_groups_asym(W, 64)
    assert sig[3, 1] == 1.0  # constant group: unit scale
    rec = OA.dequant(Q, sig, z, 64)[3, 64:128]
    assert np.all(np.abs(rec - 0.0125) <= 0.0125 * 2.0 ** -8)
    for k in (-6, 5):
        Qk, sk, zk, _ = OA.quant_groups_asym(np.ldexp(W, k).astype(np.float32), 64)
        nonconst = np.ones_like(sig, dtype=bool)
        nonconst[3, 1] = False
        np.testing.assert_array_equal(sk[nonconst], np.ldexp(sig, k)[nonconst])
        np.testing.assert_array_equal(zk[nonconst], z[nonconst])
        np.testing.assert_array_equal(Qk.reshape(6, 4, 64)[nonconst], Q.reshape(6, 4, 64)[nonconst])


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.0078125, 1.01171875, -3.0000001, 1e-3], np.float32)
    r = OA.bf16_rne(x)
    for a, b in zip(x, r):
        # nearest bfloat16 (8 significant bits), ties to even
        m, e = math.frexp(float(a))
        q = math.ldexp(round(m * 256), e - 8)
        assert float(b) == q


def test_offset_identity_and_product():
    rng = np.random.default_rng(4)
    M, K, N, g = 3, 128, 5, 64
    W = (rng.standard_normal((N, K)) * 0.02 + 0.01).astype(np.float32)
    Q, sig, z, _ = OA.quant_groups_asym(W, g)
    C = OA.correction(sig, z)
    qa = rng.integers(-7, 8, (M, K))
    alpha = rng.uniform(0.01, 0.1, M).astype(np.float32)
    mean = rng.standard_normal(M).astype(np.float32)
    w1 = rng.standard_normal(N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    y, S = OA.linear_asym(alpha, qa, Q, sig, C, g, mean, w1, b)
    for t in range(M):
        for o in range(N):
            # exact: sum_g sigma (acc_g) - C_g p_g with integer acc and p
            ref = Fraction(0)
            for gg in range(K // g):
                ks = range(gg * g, (gg + 1) * g)
                acc = sum(int(qa[t, k]) * (int(Q[o, k]) - 8) for k in ks)
                p = sum(int(qa[t, k]) for k in ks)
                ref += Fraction(float(sig[o, gg])) * acc - Fraction(float(C[o, gg])) * p
            ref = Fraction(float(alpha[t])) * ref + Fraction(float(mean[t])) * Fraction(float(w1[o])) + Fraction(float(b[o]))
            assert float(y[t, o]) == np.float32(float(ref))
            # the stored offset: the same product over the dequantized grid
            # sigma (Q - z), up to the rounding of C
            deq = sum(float(alpha[t]) * int(qa[t, k]) * float(sig[o, k // g]) * (int(Q[o, k]) - float(z[o, k // g]))
                      for k in range(K))
            deq += float(mean[t]) * float(w1[o]) + float(b[o])
            slack = float(alpha[t]) * sum(abs(sum(int(qa[t, k]) for k in range(gg * g, (gg + 1) * g))) *
                                          abs(float(sig[o, gg])) * abs(float(z[o, gg]) - 8) * 2.0 ** -22
                                          for gg in range(K // g))
            assert abs(float(y[t, o]) - deq) <= slack + 2.0 ** -22 * S[t, o]


def test_group_sums():
    qa = np.arange(-64, 64).reshape(1, 128) % 15 - 7
    p = OA.group_sums(qa, 64)
    assert p.shape == (1, 2) and p[0, 0] == qa[0, :64].sum() and p[0, 1] == qa[0, 64:].sum()
    assert np.array_equal(OQ.unpack_int4(OQ.pack_int4(np.arange(16) - 8)), np.arange(16) - 8)
