"""Factorised Paley x Sylvester rotation for any width, with zero padding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Parity pins: tests/test_oracle_kron.py.

Sources:
  CentriQ Sec. 3 "Hadamard rotation": Hadamard matrices exist at orders 2^k
  (Sylvester), q + 1 for a prime power q = 3 (mod 4) and 2 (q + 1) for
  q = 1 (mod 4) (Paley), and the Kronecker product of two is Hadamard.
  CentriQ Sec. 4.2 "Rotation" and App. B.1: H = (H_m (x) H_{2^k}) / sqrt(n')
  of order n' = m 2^k with m in {1, 12, 36, 44}; when the width n is not of
  that form the centred token is zero-padded by P = [I_n; 0] to the smallest
  admissible n' > n; the weight absorbs W P^T H^T; the product is applied as
  vec(H_{2^k} X H_m^T) with the token reshaped to X in R^{2^k x m}, at
  n'(m + 2^k) operations; centering precedes padding.

Readings where the pages are silent or garbled:
  * H_12 and H_44 are Paley type I (q = 11, 43); H_36 is Paley type II
    (q = 17).  App. B.1 calls H_36 "type I", which no prime power allows
    (35 is not one); 36 = 2 (17 + 1) is the type II order;
  * Paley matrices in their textbook form: chi the quadratic character mod q,
    Jacobsthal Q[i][j] = chi(j - i); type I: H = I + S with
    S = [[0, 1^T], [-1, Q]]; type II: C = [[0, 1^T], [1, Q]] and
    H = [[C + I, C - I], [C - I, -C - I]]; the border row and column come first;
  * vec stacks columns: X[r][c] = x[c 2^k + r], so each column is a
    contiguous block of 2^k coordinates;
  * canonical float32 order: pad, the Sylvester factor on every block as the
    un-normalised staged transform of oracle.hadamard (strides 1, 2, ...,
    each butterfly rounded once), then for each output the m-term sum
    sum_c H_m[c'][c] u[c 2^k + r] taken in increasing c (each addition
    rounded once), then one multiplication by RN32(1 / sqrt(n'));
  * the smallest admissible n' >= n is taken over all k >= 0.
"""
from __future__ import annotations

import math

import numpy as np

from .hadamard import fwht_fp32_canonical, sylvester

ORDERS = (1, 12, 36, 44)


def quadratic_character(q: int) -> np.ndarray:
    """chi(a) for a = 0 .. q-1 (q prime): 0, +1 on nonzero squares, -1 else."""
    chi = -np.ones(q, dtype=np.int64)
    chi[0] = 0
    for a in range(1, q):
        chi[(a * a) % q] = 1
    return chi


def jacobsthal(q: int) -> np.ndarray:
    chi = quadratic_character(q)
    i = np.arange(q)
    return chi[(i[None, :] - i[:, None]) % q]


def paley_i(q: int) -> np.ndarray:
    """Order q + 1, q = 3 (mod 4): H = I + [[0, 1^T], [-1, Q]]."""
    assert q % 4 == 3
    n = q + 1
    S = np.zeros((n, n), dtype=np.int64)
    S[0, 1:] = 1
    S[1:, 0] = -1
    S[1:, 1:] = jacobsthal(q)
    return np.eye(n, dtype=np.int64) + S


def paley_ii(q: int) -> np.ndarray:
    """Order 2 (q + 1), q = 1 (mod 4): from C = [[0, 1^T], [1, Q]]."""
    assert q % 4 == 1
    n = q + 1
    C = np.zeros((n, n), dtype=np.int64)
    C[0, 1:] = 1
    C[1:, 0] = 1
    C[1:, 1:] = jacobsthal(q)
    I = np.eye(n, dtype=np.int64)
    return np.block([[C + I, C - I], [C - I, -C - I]])


def hadamard_m(m: int) -> np.ndarray:
    if m == 1:
        return np.ones((1, 1), dtype=np.int64)
    if m == 12:
        return paley_i(11)
    if m == 44:
        return paley_i(43)
    if m == 36:
        return paley_ii(17)
    raise ValueError("m must be 1, 12, 36 or 44")


def admissible(n: int):
    """(m, 2^k, n') with n' = m 2^k the smallest admissible order >= n."""
    best = None
    for m in ORDERS:
        b = 1
        while m * b < n:
            b *= 2
        if best is None or m * b < best[2]:
            best = (m, b, m * b)
    return best


def rotation_matrix(m: int, b: int) -> np.ndarray:
    """(H_m (x) H_b) / sqrt(m b) as a dense float64 matrix (brute force)."""
    return np.kron(hadamard_m(m).astype(np.float64), sylvester(b)) / math.sqrt(m * b)


def pad(x: np.ndarray, npad: int) -> np.ndarray:
    x = np.asarray(x)
    out = np.zeros(x.shape[:-1] + (npad,), dtype=x.dtype)
    out[..., : x.shape[-1]] = x
    return out


def rotate_fp64(x: np.ndarray, m: int, b: int) -> np.ndarray:
    """H P x in float64 via vec(H_b X H_m^T), X[r][c] = x[c b + r]."""
    x = pad(np.asarray(x, dtype=np.float64), m * b)
    lead = x.shape[:-1]
    X = x.reshape(lead + (m, b))                       # [.., c, r] = X[r][c]
    Hb = sylvester(b)
    Hm = hadamard_m(m).astype(np.float64)
    Y = np.einsum("rs,...cs->...cr", Hb, X)            # H_b applied to every column
    Y = np.einsum("dc,...cr->...dr", Hm, Y)            # then X H_m^T across columns
    return Y.reshape(lead + (m * b,)) / math.sqrt(m * b)


def rotate_fp32(x32: np.ndarray, m: int, b: int) -> np.ndarray:
    """The canonical float32 order (see the module docstring)."""
    v = pad(np.asarray(x32, dtype=np.float32), m * b)
    u = fwht_fp32_canonical(v, b, scale=False)
    lead = u.shape[:-1]
    U = u.reshape(lead + (m, b))
    Hm = hadamard_m(m)
    W = np.empty_like(U)
    for cp in range(m):
        acc = U[..., 0, :] * np.float32(Hm[cp, 0])
        for c in range(1, m):
            acc = (acc + U[..., c, :] * np.float32(Hm[cp, c])).astype(np.float32)
        W[..., cp, :] = acc
    cn = np.float32(1.0 / math.sqrt(m * b))
    return (W.reshape(lead + (m * b,)) * cn).astype(np.float32)
