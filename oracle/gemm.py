"""Grouped integer products, the fp32-scale epilogue and the MXFP4 product.

Parity pins: tests/test_oracle_gemm.py.

Sources:
  CentriQ Sec. 4.2, Eq. 5: y_t = W_R Q_a(H P x_t^c) + xbar_t w_1 + b, with the
  rank-1 term and the bias added in the epilogue of the 4-bit product;
  App. B.2, Eq. 9: the same epilogue in the fused kernel.
  Per-group weight scales along the input dimension: CentriQ Sec. 3 Eq. 2
  (groups of g consecutive input columns, one scale per row and group).
  WUSH review, "Core claim" / Fig. 2 caption: MXFP4 GEMM with G = 32.

The integer group sums acc_g[t, o] = sum_{k in group g} qa[t, k] qw[o, k] are
exact; they are formed with float64 matrix products, which are exact for
integers while every partial sum stays below 2^53 (checked).
"""
from __future__ import annotations

import numpy as np


def group_acc(qa: np.ndarray, qw: np.ndarray, group: int) -> np.ndarray:
    """int64 [K/group, M, N] exact group sums."""
    qa = np.asarray(qa, dtype=np.float64)
    qw = np.asarray(qw, dtype=np.float64)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and K % group == 0
    bound = group * np.max(np.abs(qa), initial=0) * np.max(np.abs(qw), initial=0)
    assert bound < 2.0 ** 53
    G = K // group
    out = np.empty((G, M, N), dtype=np.int64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        out[g] = np.rint(qa[:, sl] @ qw[:, sl].T).astype(np.int64)
    return out


def epilogue_int(alpha, acc, w_scale, mean=None, w1=None, bias=None):
    """y* = RN32(alpha_t sum_g s_w[o,g] acc_g[t,o] + m_t w1[o] + b[o]) in
    float64 before the single rounding.  Also returns S, the sum of the
    magnitudes of every term, which bounds float32 rounding error of any
    evaluation order."""
    alpha = np.asarray(alpha, dtype=np.float64)
    sw = np.asarray(w_scale, dtype=np.float64)       # [N, G]
    G = acc.shape[0]
    F = np.zeros(acc.shape[1:], dtype=np.float64)
    Fa = np.zeros(acc.shape[1:], dtype=np.float64)
    for g in range(G):
        term = sw[:, g][None, :] * acc[g].astype(np.float64)
        F += term
        Fa += np.abs(term)
    y = alpha[:, None] * F
    S = np.abs(alpha)[:, None] * Fa
    if mean is not None:
        r1 = np.asarray(mean, dtype=np.float64)[:, None] * np.asarray(w1, dtype=np.float64)[None, :]
        y = y + r1
        S = S + np.abs(r1)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)[None, :]
        y = y + b
        S = S + np.abs(b)
    return y.astype(np.float32), S


def gemm_mx(a_val: np.ndarray, w_val: np.ndarray, bias=None):
    """MXFP4 product from dequantized values (each E2M1 value times its
    block's power of two), float64, then one rounding; returns (y*, S)."""
    A = np.asarray(a_val, dtype=np.float64)
    W = np.asarray(w_val, dtype=np.float64)
    y = A @ W.T
    S = np.abs(A) @ np.abs(W).T
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)[None, :]
        y = y + b
        S = S + np.abs(b)
    return y.astype(np.float32), S


def bf16_ulp(y: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |y| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(y, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def output_tolerance(y_ref: np.ndarray, S: np.ndarray, n_terms: int) -> np.ndarray:
    """Allowed |y_gpu - y*| for a bfloat16 output: one bfloat16 ulp of y*
    (the output rounding) plus (n_terms + 3) float32 unit roundoffs of S
    (an fp32 sum of n_terms scaled partial sums plus the epilogue's
    multiply and adds, in any order)."""
    return bf16_ulp(y_ref) + (n_terms + 3) * 2.0 ** -24 * np.asarray(S, dtype=np.float64)
