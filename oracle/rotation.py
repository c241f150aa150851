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


def dense32_fp32(x: np.ndarray, T: np.ndarray) -> np.ndarray:
    """The per-block transform rounded once to float32.  With bfloat16 T and
    bfloat16 x every product has at most 16 significant bits and a 32-term sum
    is exact in float64, so this is the correctly rounded value."""
    return dense32_fp64(x, T).astype(np.float32)
