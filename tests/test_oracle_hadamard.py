"""Pins of oracle/hadamard.py against the pages and the mathematics (CPU only)."""
import numpy as np
import pytest
from scipy.linalg import hadamard as scipy_hadamard

from conftest import read_golden
from oracle import hadamard as H

POW2 = [1, 2, 4, 8, 32, 128, 1024]


@pytest.mark.parametrize("h", POW2)
def test_sylvester_matches_library(h):
    # special case reducing to a library routine: scipy builds the same
    # Sylvester construction by repeated Kronecker blocks
    np.testing.assert_array_equal(H.sylvester(h), scipy_hadamard(h).astype(np.float64))


def test_sylvester_h8_golden():
    rows = [[float(t) for t in ln.split()] for ln in read_golden("sylvester_h8.txt")]
    np.testing.assert_array_equal(H.sylvester(8), np.array(rows))


@pytest.mark.parametrize("h", [2, 16, 256, 1024])
def test_kronecker_recursion(h):
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    np.testing.assert_array_equal(H.sylvester(h), np.kron(h2, H.sylvester(h // 2)))


@pytest.mark.parametrize("h", [4, 64, 1024])
def test_orthogonality_and_row_sums(h):
    # CentriQ Sec. 3: H_n H_n^T = n I; proof of Lemma 1: one row of the
    # Sylvester matrix sums to 2^k, every other row to zero
    S = H.sylvester(h)
    np.testing.assert_array_equal(S @ S.T, h * np.eye(h))
    rs = S.sum(axis=1)
    assert rs[0] == h and np.all(rs[1:] == 0)


@pytest.mark.parametrize("h", [32, 128, 1024])
def test_dense_block_transform(h):
    rng = np.random.default_rng(1)
    d = 3 * h
    x = rng.standard_normal((5, d))
    v = H.block_hadamard_fp64(x, h)
    # basis vector -> column of H / sqrt h, inside its own block only
    e = np.zeros(d)
    e[h + 3] = 1.0
    ve = H.block_hadamard_fp64(e, h)
    assert np.all(ve[:h] == 0) and np.all(ve[2 * h:] == 0)
    np.testing.assert_allclose(ve[h:2 * h], H.sylvester(h)[:, 3] / np.sqrt(h), rtol=0, atol=1e-15)
    # orthogonal and symmetric: norm kept, applying twice returns the input
    np.testing.assert_allclose(np.linalg.norm(v, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(H.block_hadamard_fp64(v, h), x, rtol=0, atol=1e-12)
    # DC: the all-ones block maps onto its first coordinate, magnitude sqrt h
    ones = H.block_hadamard_fp64(np.ones(d), h).reshape(3, h)
    np.testing.assert_allclose(ones[:, 0], np.sqrt(h), rtol=1e-14)
    assert np.max(np.abs(ones[:, 1:])) < 1e-12


@pytest.mark.parametrize("h", [32, 128, 1024])
def test_unnormalised_fwht_twice_is_h_times_identity(h):
    rng = np.random.default_rng(2)
    x = rng.integers(-50, 50, size=(3, 2 * h)).astype(np.float32)
    # integer inputs stay exact in float32 through an unnormalised transform
    y = H.fwht_fp32_canonical(x, h) / H.scale_fp32(h)
    z = H.fwht_fp32_canonical(y, h) / H.scale_fp32(h)
    if h in (32, 128):  # c_h not a power of two: undo with float64 and round
        np.testing.assert_allclose(z, h * x, rtol=1e-5)
    else:
        np.testing.assert_array_equal(z, h * x)


@pytest.mark.parametrize("h", [32, 128, 512, 1024])
def test_canonical_fp32_close_to_fp64(h):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 2 * h)).astype(np.float32)
    v32 = H.fwht_fp32_canonical(x, h).astype(np.float64)
    v64 = H.block_hadamard_fp64(x.astype(np.float64), h)
    # each output is a signed sum of h inputs, log2(h) roundings deep
    bound = (np.log2(h) + 1) * 2.0 ** -24 * np.sqrt(h) * np.max(np.abs(x)) * 2
    assert np.max(np.abs(v32 - v64)) <= bound


def test_canonical_stage_order_golden():
    ln = read_golden("fwht_order_h4.txt")
    x = np.array([float(t) for t in ln[0].split()[1:]], dtype=np.float32)
    want = np.array([float(t) for t in ln[1].split()[1:]], dtype=np.float64)
    got = H.fwht_fp32_canonical(x[None, :], 4)[0].astype(np.float64)
    np.testing.assert_array_equal(got, want)


def test_scale_constant():
    for h in [32, 128, 512, 1024]:
        c = H.scale_fp32(h)
        assert c == np.float32(1.0 / np.sqrt(h))
        # correctly rounded: no other float32 is nearer to 1/sqrt(h)
        exact = 1.0 / np.sqrt(np.longdouble(h))
        up = np.nextafter(c, np.float32(1))
        dn = np.nextafter(c, np.float32(0))
        assert abs(np.longdouble(c) - exact) <= abs(np.longdouble(up) - exact)
        assert abs(np.longdouble(c) - exact) <= abs(np.longdouble(dn) - exact)
