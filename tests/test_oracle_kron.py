"""Pins of the Paley x Sylvester rotation oracle (oracle/kron.py):
- the Hadamard property of H_12, H_36, H_44, and the quadratic residues against
  Euler's criterion;
- the Kronecker identity against np.kron, and orthogonality;
- the closed form the page states for H 1_n at native width;
- the DC property of centred, padded tokens;
- m = 1 reducing to the plain Sylvester transform;
- the float32 order within its rounding bound of float64;
- the admissible orders by brute-force enumeration."""
import math

import numpy as np
import pytest

from oracle import hadamard as OH
from oracle import kron as KR


@pytest.mark.parametrize("m", [12, 36, 44])
def test_paley_matrices_are_hadamard(m):
    H = KR.hadamard_m(m)
    assert set(np.unique(H)) == {-1, 1}
    np.testing.assert_array_equal(H @ H.T, m * np.eye(m, dtype=np.int64))


@pytest.mark.parametrize("q", [11, 17, 43])
def test_quadratic_character_euler(q):
    chi = KR.quadratic_character(q)
    for a in range(1, q):
        e = pow(a, (q - 1) // 2, q)  # Euler's criterion: 1 for residues, q - 1 otherwise
        assert chi[a] == (1 if e == 1 else -1)
    assert chi[0] == 0
    # the residues of 11 and 17 as usually listed
    if q == 11:
        assert set(np.flatnonzero(chi == 1)) == {1, 3, 4, 5, 9}
    if q == 17:
        assert set(np.flatnonzero(chi == 1)) == {1, 2, 4, 8, 9, 13, 15, 16}


@pytest.mark.parametrize("m,b", [(12, 16), (36, 32), (44, 16), (1, 64), (12, 64)])
def test_kronecker_identity_and_orthogonality(m, b):
    R = KR.rotation_matrix(m, b)
    np.testing.assert_allclose(R @ R.T, np.eye(m * b), atol=1e-12)
    rng = np.random.default_rng(m + b)
    x = rng.standard_normal((3, m * b - 5))   # padded by 5
    want = (R @ KR.pad(x, m * b).T).T
    np.testing.assert_allclose(KR.rotate_fp64(x, m, b), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("m,b", [(12, 16), (36, 32), (44, 64)])
def test_ones_map_to_first_coordinates(m, b):
    # at native width H 1_n = sqrt(2^k / m) (H_m 1_m) (x) e_1
    y = KR.rotate_fp64(np.ones(m * b), m, b)
    hm1 = KR.hadamard_m(m).sum(axis=1).astype(np.float64)
    want = np.zeros(m * b)
    want[::b] = math.sqrt(b / m) * hm1
    np.testing.assert_allclose(y, want, atol=1e-12)


def test_centred_padded_token_has_no_dc():
    m, b = KR.admissible(1920)[:2]
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1920) + 3.0
    xc = x - x.mean()
    y = KR.rotate_fp64(xc, m, b)
    h1 = KR.rotate_fp64(np.ones(m * b), m, b)   # H 1_{n'}
    assert abs(y @ h1) < 1e-9
    assert abs(np.linalg.norm(y) - np.linalg.norm(xc)) < 1e-9


def test_m1_is_plain_sylvester():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    np.testing.assert_array_equal(KR.rotate_fp32(x, 1, 256), OH.fwht_fp32_canonical(x, 256))


@pytest.mark.parametrize("n", [1152, 1920, 2240, 3072, 2816])
def test_fp32_order_within_rounding(n):
    m, b, npad = KR.admissible(n)
    rng = np.random.default_rng(n)
    x = (rng.standard_normal((3, n)) * 2).astype(np.float32)
    y32 = KR.rotate_fp32(x, m, b).astype(np.float64)
    y64 = KR.rotate_fp64(x.astype(np.float64), m, b)
    # each output: log2(b) butterflies and m - 1 additions on partial sums
    # bounded by sqrt(n') |x|_2, then one multiply
    bound = (math.log2(b) + m + 2) * 2.0 ** -24 * np.linalg.norm(x, axis=1, keepdims=True)
    assert np.all(np.abs(y32 - y64) <= bound)


def test_admissible_by_enumeration():
    for n in [16, 100, 700, 1000, 1152, 1500, 1920, 2048, 2240, 3000, 3072, 3840, 4608, 5120, 6000, 12288]:
        cands = sorted(m * 2 ** k for m in KR.ORDERS for k in range(0, 16) if m * 2 ** k >= n)
        m, b, npad = KR.admissible(n)
        assert npad == cands[0] and m * b == npad and b & (b - 1) == 0
