"""Randomised permuted block-Hadamard (RPBH) rotation and per-32 dense transforms.

Parity pins: tests/test_oracle_rotation.py.

Sources:
  OrbitQuant PR #25, "Default changes": extra RPBH rounds are independent
  rounds of the same construction; "Runtime work": dense block-Hadamard matrix
  form, blocks <= 1024.
  CentriQ, related-work paragraph on OrbitQuant: weights and activations are
  quantized in a randomly permuted block-Hadamard basis; Sec. 3 "Hadamard
  rotation": W x = (W H^T)(H x).
  FLUX.1-schnell-OrbitQuant-W4A4 model card, "Quantization" and "Artifact
  Files": rotation "rpbh" with deterministic stored rotation metadata.
  WUSH review, "Core claim": one transform per quantization block, activations
  take T_x, weights its inverse-transpose.

Reading (the pages do not spell the round out): one round is
R_r = B_h D_{s_r} P_{pi_r}: gather (P_pi v)_i = v_{pi(i)} over the whole
width d, multiply by the +-1 signs s_r, then the normalised block Hadamard
B_h.  Two rounds compose as R = R_2 R_1.
"""
from __future__ import annotations

import math

import numpy as np

from .hadamard import block_hadamard_fp64, fwht_fp32_canonical, sylvester


def rpbh_fp64(x: np.ndarray, perm: np.ndarray, signs: np.ndarray, h: int) -> np.ndarray:
    """R x in float64 for every row of x (last axis = d)."""
    v = np.asarray(x, dtype=np.float64)
    for r in range(perm.shape[0]):
        u = v[..., perm[r]] * signs[r].astype(np.float64)
        v = block_hadamard_fp64(u, h)
    return v


def rpbh_fp32(x32: np.ndarray, perm: np.ndarray, signs: np.ndarray, h: int) -> np.ndarray:
    """R x in the canonical float32 order (the gather and the sign flips are
    exact; each round's Hadamard follows ``fwht_fp32_canonical``)."""
    v = np.asarray(x32, dtype=np.float32)
    for r in range(perm.shape[0]):
        u = v[..., perm[r]] * signs[r].astype(np.float32)
        v = fwht_fp32_canonical(u, h)
    return v


def rpbh_matrix(perm: np.ndarray, signs: np.ndarray, h: int) -> np.ndarray:
    """The whole rotation as an explicit d x d float64 matrix (brute force)."""
    d = perm.shape[1]
    R = np.eye(d)
    Hb = np.kron(np.eye(d // h), sylvester(h) / np.sqrt(float(h)))
    for r in range(perm.shape[0]):
        P = np.zeros((d, d))
        P[np.arange(d), perm[r]] = 1.0
        R = Hb @ np.diag(signs[r].astype(np.float64)) @ P @ R
    return R


def dense32_fp64(x: np.ndarray, T: np.ndarray) -> np.ndarray:
    """v_b = T_b x_b for each consecutive 32-block b of the last axis."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    nb = d // 32
    xb = x.reshape(x.shape[:-1] + (nb, 32))
    v = np.einsum("bij,...bj->...bi", np.asarray(T, dtype=np.float64), xb)
    return v.reshape(x.shape)


def dense32_weight_transform(t_bits: np.ndarray) -> np.ndarray:
    """Weight side of the per-block pair (WUSH review, "Core claim": the
    weights take the inverse-transpose of the activation transform,
    T_w = T_x^{-T}), formed in float64 from the stored bfloat16 matrices:
    returns float64 [nb][32][32] with T_w,b = (T_b^{-1})^T."""
    T = (np.asarray(t_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.transpose(np.linalg.inv(T), (0, 2, 1))


def _exponent(a: np.ndarray) -> np.ndarray:
    """floor(log2 |a|) of the nonzero entries (float64 array), NaN at zeros."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, np.nan)))
    return e


def _rn32_scaled_int(n: int, e: int) -> np.float32:
    """RN32 (ties to even) of the exact value n * 2^e (Python integers)."""
    if n == 0:
        return np.float32(0.0)
    sign = -1 if n < 0 else 1
    n = abs(n)
    lsb = max(n.bit_length() + e - 24, -149)   # weight of the last kept bit
    shift = lsb - e
    if shift > 0:
        q, r = divmod(n, 1 << shift)
        half = 1 << (shift - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
    else:
        q = n << (-shift)
    return np.float32(sign * math.ldexp(q, lsb))


def _bf16_parts(a: float):
    """(integer mantissa, exponent) with a = m * 2^e exactly (a float)."""
    m, e = math.frexp(a)
    return int(m * (1 << 53)), e - 53


def dense32_fp32(x32: np.ndarray, T: np.ndarray):
    """v_b = T_b x_b per 32-block rounded once to float32: the exact sum of the
    exact products, then RN32.

    With bfloat16 T and x each product has at most 16 significant bits, so a
    32-term float64 sum is exact whenever the exponents floor(log2 |T_ij x_j|)
    of one output's nonzero products span at most 32 (every partial sum is then
    a multiple of the smallest product's last bit below 2^53 of them).  That is
    checked for every output; the rest are summed exactly in integers.  Returns
    (v float32, number of outputs summed in integers)."""
    x = np.asarray(x32, dtype=np.float64)
    Tm = np.asarray(T, dtype=np.float64)
    v = dense32_fp64(x, Tm).astype(np.float32)
    d = x.shape[-1]
    xr = x.reshape(-1, d // 32, 32)
    vr = v.reshape(-1, d // 32, 32)
    eT = _exponent(Tm)                                   # [nb, 32, 32]
    ex = _exponent(xr)                                   # [rows, nb, 32]
    # conservative span per (row, block, output): largest exponent sum minus
    # smallest, each bounded separately
    tmax, tmin = np.nanmax(eT, axis=-1, initial=-np.inf), np.nanmin(eT, axis=-1, initial=np.inf)
    xmax, xmin = np.nanmax(ex, axis=-1, initial=-np.inf), np.nanmin(ex, axis=-1, initial=np.inf)
    loose = (xmax[:, :, None] + tmax[None]) - (xmin[:, :, None] + tmin[None])
    suspect = np.argwhere(loose > 32)
    exact_int = 0
    for r, b in {(int(r), int(b)) for r, b, _ in suspect}:
        span = ex[r, b][None, :] + eT[b]                 # [32 outputs, 32 terms]
        hi = np.nanmax(span, axis=-1, initial=-np.inf)
        lo = np.nanmin(span, axis=-1, initial=np.inf)
        for i in np.nonzero(hi - lo > 32)[0]:
            parts = [(_bf16_parts(float(Tm[b, i, j])), _bf16_parts(float(xr[r, b, j])))
                     for j in range(32) if Tm[b, i, j] != 0 and xr[r, b, j] != 0]
            if not parts:
                continue
            emin = min(pt[1] + px[1] for pt, px in parts)
            n = sum(pt[0] * px[0] << (pt[1] + px[1] - emin) for pt, px in parts)
            vr[r, b, i] = _rn32_scaled_int(n, emin)
            exact_int += 1
    return v, exact_int
