"""Asymmetric grouped INT4 weights and the product that consumes them.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Parity pins: tests/test_oracle_asym.py.

Sources:
  CentriQ Sec. 3 "Preliminaries", Eq. 2: weights on an asymmetric b-bit grid
  per group of g consecutive input columns, W_g = sigma (Q_g - z) with
  Q_g in {0 .. 2^b - 1} and a per-(row, group) scale sigma and shift z stored
  in 16 bits; round-to-nearest (RTN) sets both from the group's minimum and
  maximum.
  CentriQ App. B.2 ("fused kernel"): codes are stored as Q - 8 with zero point
  z' = z - 8, which leaves a correction C = sigma z' per row and 64-column
  group; it is absorbed through the activation columns alpha_t p_t, with p_t
  the group sums of the activation codes, so the integer main product is
  unchanged.  App. B.3 (Table 3): groups of 64, 16-bit scale and zero point
  in the model precision.

Readings where the pages are silent:
  * the 16-bit format is bfloat16 (the model precision of the pages' DiTs);
  * RTN min-max: r = RN32(max - min); sigma = RNbf16(RN32(r / 15)) for r > 0,
    sigma = 1 for a constant group; z = RNbf16(RN32(-min / sigma)), a real
    shift (not rounded to an integer);
  * Q = clamp(RNE(RN32(RN32(w / sigma) + z)), 0, 15); stored codes Q - 8 as
    4-bit two's complement (element 2i in bits 3..0);
  * C = RN32(sigma RN32(z - 8)), the stored correction;
  * y* = RN32(float64(alpha_t sum_g (sigma_g acc_g - C_g p_g) + m_t w1 + b))
    with acc_g = sum_{k in g} q_a q' (q' = Q - 8) and p_g = sum_{k in g} q_a,
    both exact integers.
"""
from __future__ import annotations

import numpy as np


def bf16_rne(x) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def quant_groups_asym(w32: np.ndarray, group: int):
    """(Q int64 [N, K] in 0..15, sigma float32 [N, G], z float32 [N, G], flags)
    with sigma and z bfloat16 values; flags mark elements whose pre-rounding
    value lies within 1e-6 (relative) of a half-integer."""
    w32 = np.asarray(w32, dtype=np.float32)
    N, K = w32.shape
    G = K // group
    g = w32.reshape(N, G, group)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    r = (mx - mn).astype(np.float32)
    sig = np.where(r > 0, bf16_rne((r / np.float32(15)).astype(np.float32)), np.float32(1.0)).astype(np.float32)
    z = bf16_rne((-mn / sig).astype(np.float32))
    t = ((g / sig[..., None]).astype(np.float32) + z[..., None]).astype(np.float32)
    Q = np.clip(np.rint(t), 0, 15).astype(np.int64)
    frac = np.abs(t.astype(np.float64) - np.floor(t.astype(np.float64)) - 0.5)
    flags = frac <= 1e-6 * np.abs(t.astype(np.float64))
    return Q.reshape(N, K), sig, z, flags.reshape(N, K)


def correction(sig: np.ndarray, z: np.ndarray) -> np.ndarray:
    """C = RN32(sigma RN32(z - 8))."""
    zp = (np.asarray(z, np.float32) - np.float32(8)).astype(np.float32)
    return (np.asarray(sig, np.float32) * zp).astype(np.float32)


def dequant(Q, sig, z, group: int) -> np.ndarray:
    """sigma (Q - z) in float64 (the grid value of Eq. 2)."""
    s = np.repeat(np.asarray(sig, np.float64), group, axis=1)
    zz = np.repeat(np.asarray(z, np.float64), group, axis=1)
    return s * (np.asarray(Q, np.float64) - zz)


def group_sums(qa: np.ndarray, group: int) -> np.ndarray:
    """p[t, g] = sum of the activation codes of group g (exact integers)."""
    qa = np.asarray(qa, dtype=np.int64)
    M, K = qa.shape
    return qa.reshape(M, K // group, group).sum(axis=-1)


def linear_asym(alpha, qa, Q, sig, C, group: int, mean=None, w1=None, bias=None):
    """y* = RN32(alpha_t sum_g (sigma_g acc_g - C_g p_g) + m_t w1 + b), float64
    before the one rounding, and S, the sum of the terms' magnitudes."""
    qa = np.asarray(qa, dtype=np.int64)
    qp = np.asarray(Q, dtype=np.int64) - 8
    M, K = qa.shape
    G = K // group
    p = group_sums(qa, group).astype(np.float64)          # [M, G]
    sig = np.asarray(sig, np.float64)
    C = np.asarray(C, np.float64)
    F = np.zeros((M, qp.shape[0]))
    Fa = np.zeros_like(F)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        acc = qa[:, sl].astype(np.float64) @ qp[:, sl].T.astype(np.float64)   # exact: |acc| < 2^53
        t1 = sig[:, g][None, :] * acc
        t2 = C[:, g][None, :] * p[:, g][:, None]
        F += t1 - t2
        Fa += np.abs(t1) + np.abs(t2)
    a = np.asarray(alpha, np.float64)[:, None]
    y = a * F
    S = np.abs(a) * Fa
    if mean is not None:
        r1 = np.asarray(mean, np.float64)[:, None] * np.asarray(w1, np.float64)[None, :]
        y = y + r1
        S = S + np.abs(r1)
    if bias is not None:
        b = np.asarray(bias, np.float64)[None, :]
        y = y + b
        S = S + np.abs(b)
    return y.astype(np.float32), S
