"""Sylvester-Hadamard matrices and the block Walsh-Hadamard transform.

Parity pins: tests/test_oracle_hadamard.py.

Sources:
  CentriQ, Sec. 3 "Hadamard rotation": H_n in {+-1}^{n x n} with
  H_n H_n^T = n I, so H = H_n / sqrt(n) is orthogonal; Sylvester matrices
  exist at every order 2^k.  Proof of Lemma 1 (appendix): one row of the
  Sylvester matrix sums to 2^k and every other row to zero.
  OrbitQuant PR #25, "Runtime work": the pre-rotation is equivalent to a dense
  block-Hadamard matrix product with blocks of at most 1024.
"""
from __future__ import annotations

import numpy as np


def popcount(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, dtype=np.int64)
    c = np.zeros_like(a)
    while np.any(a):
        c += a & 1
        a = a >> 1
    return c


def sylvester(h: int) -> np.ndarray:
    """Unnormalised Sylvester matrix of order h = 2^k as float64.

    Entry (i, j) is (-1)^{popcount(i AND j)}, the closed form of the
    Kronecker-power construction [[1, 1], [1, -1]]^{(x) k}."""
    if h < 1 or h & (h - 1):
        raise ValueError("h must be a power of two")
    i = np.arange(h)
    return np.where(popcount(i[:, None] & i[None, :]) % 2 == 0, 1.0, -1.0)


def block_hadamard_fp64(u: np.ndarray, h: int) -> np.ndarray:
    """Normalised block Hadamard in float64: every consecutive block of h
    coordinates b of the last axis becomes (1/sqrt h) H_h b.

    Written as the dense matrix product the OrbitQuant export uses."""
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    if d % h:
        raise ValueError("d must be a multiple of h")
    H = sylvester(h) / np.sqrt(float(h))
    blocks = u.reshape(u.shape[:-1] + (d // h, h))
    return (blocks @ H.T).reshape(u.shape)


def scale_fp32(h: int) -> np.float32:
    """c_h = 1/sqrt(h) rounded to the nearest float32."""
    return np.float32(1.0 / np.sqrt(float(h)))


def fwht_fp32_canonical(u: np.ndarray, h: int, scale: bool = True) -> np.ndarray:
    """Block Walsh-Hadamard in the canonical float32 order.

    The pages fix the matrix but not the evaluation order; the order used to
    define float32 results (and therefore the integer codes) is: butterfly
    stages with strides 1, 2, 4, ..., h/2 in that order, each butterfly
    (a, b) -> (a + b, a - b) rounded once to float32, then one float32
    multiplication of every output by c_h = RN32(1/sqrt h) (left out with
    scale=False, for transforms that normalise once at the end)."""
    u = np.asarray(u, dtype=np.float32)
    d = u.shape[-1]
    if d % h:
        raise ValueError("d must be a multiple of h")
    lead = u.shape[:-1]
    a = u.reshape(lead + (d // h, h)).copy()
    s = 1
    while s < h:
        v = a.reshape(lead + (d // h, h // (2 * s), 2, s))
        lo = v[..., 0, :]
        hi = v[..., 1, :]
        out = np.empty_like(v)
        out[..., 0, :] = lo + hi
        out[..., 1, :] = lo - hi
        a = out.reshape(lead + (d // h, h))
        s *= 2
    if scale:
        a = a * scale_fp32(h)
    return a.reshape(u.shape).astype(np.float32)
