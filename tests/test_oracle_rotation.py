"""Pins of oracle/rotation.py (CPU only)."""
import math

import numpy as np
import pytest

from conftest import read_golden
from oracle import rotation as R
from oracle import hadamard as H


def _meta(d, rounds, seed):
    rng = np.random.default_rng(seed)
    perm = np.stack([rng.permutation(d) for _ in range(rounds)]).astype(np.int32)
    signs = np.where(rng.integers(0, 2, size=(rounds, d)) == 1, 1, -1).astype(np.int8)
    return perm, signs


def test_gather_sign_convention_golden():
    ln = read_golden("gather_sign.txt")
    vals = {l.split()[0]: [float(t) for t in l.split()[1:]] for l in ln}
    x = np.array(vals["x"])
    perm = np.array([vals["perm"]], dtype=np.int32)
    signs = np.array([vals["signs"]], dtype=np.int8)
    np.testing.assert_array_equal(R.rpbh_fp64(x, perm, signs, 1), vals["out"])
    np.testing.assert_array_equal(R.rpbh_fp32(x.astype(np.float32), perm, signs, 1), vals["out"])


@pytest.mark.parametrize("d,h,rounds", [(256, 32, 1), (384, 128, 2), (2048, 1024, 1)])
def test_fwht_path_equals_explicit_matrix(d, h, rounds):
    # OrbitQuant PR #25 "Runtime work": the rotation equals a dense
    # block-Hadamard matrix product; here built from P, D and B explicitly
    perm, signs = _meta(d, rounds, 7)
    Rm = R.rpbh_matrix(perm, signs, h)
    x = np.random.default_rng(8).standard_normal((4, d))
    np.testing.assert_allclose(R.rpbh_fp64(x, perm, signs, h), x @ Rm.T, rtol=0, atol=1e-11)
    np.testing.assert_allclose(Rm.T @ Rm, np.eye(d), rtol=0, atol=1e-12)


def test_rounds_compose():
    d, h = 512, 128
    perm, signs = _meta(d, 2, 9)
    x = np.random.default_rng(10).standard_normal((3, d))
    one = R.rpbh_fp64(R.rpbh_fp64(x, perm[:1], signs[:1], h), perm[1:], signs[1:], h)
    np.testing.assert_allclose(R.rpbh_fp64(x, perm, signs, h), one, rtol=0, atol=1e-13)
    x32 = x.astype(np.float32)
    one32 = R.rpbh_fp32(R.rpbh_fp32(x32, perm[:1], signs[:1], h), perm[1:], signs[1:], h)
    np.testing.assert_array_equal(R.rpbh_fp32(x32, perm, signs, h), one32)


def test_identity_metadata_reduces_to_block_sylvester():
    d, h = 256, 64
    perm = np.arange(d, dtype=np.int32)[None]
    signs = np.ones((1, d), dtype=np.int8)
    x = np.random.default_rng(11).standard_normal((2, d))
    np.testing.assert_allclose(R.rpbh_fp64(x, perm, signs, h), H.block_hadamard_fp64(x, h), atol=1e-14)
    # CentriQ App. B.1: the Sylvester factor sends the all-ones vector onto its
    # first coordinate; a constant token c 1 becomes c sqrt(h) e_0 per block
    c = 2.5
    v = R.rpbh_fp64(np.full(d, c), perm, signs, h).reshape(d // h, h)
    np.testing.assert_allclose(v[:, 0], c * np.sqrt(h), rtol=1e-14)
    assert np.max(np.abs(v[:, 1:])) < 1e-12


def test_two_identity_rounds_are_the_identity():
    # the normalised Sylvester block is symmetric and orthogonal, so with an
    # identity permutation and all-plus signs two rounds give back the input
    d, h = 512, 128
    perm = np.tile(np.arange(d, dtype=np.int32), (2, 1))
    signs = np.ones((2, d), dtype=np.int8)
    x = np.random.default_rng(17).standard_normal((3, d))
    np.testing.assert_allclose(R.rpbh_fp64(x, perm, signs, h), x, rtol=0, atol=1e-13)
    # and a wrong stage order or a missing scale would not: one round is not the identity
    assert np.max(np.abs(R.rpbh_fp64(x, perm[:1], signs[:1], h) - x)) > 0.1


def test_norm_and_row_sum_split():
    # CentriQ App. C.5, Eq. 10: R x = R x^c + xbar R 1 (R linear)
    d, h = 1024, 128
    perm, signs = _meta(d, 2, 12)
    x = np.random.default_rng(13).standard_normal((6, d)) + 3.0
    m = x.mean(axis=1, keepdims=True)
    lhs = R.rpbh_fp64(x, perm, signs, h)
    rhs = R.rpbh_fp64(x - m, perm, signs, h) + m * R.rpbh_fp64(np.ones(d), perm, signs, h)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(lhs, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


@pytest.mark.parametrize("d,h,rounds", [(3072, 1024, 1), (1920, 128, 2), (1024, 128, 1)])
def test_fp32_canonical_close_to_fp64(d, h, rounds):
    perm, signs = _meta(d, rounds, 14)
    x = np.random.default_rng(15).standard_normal((16, d)).astype(np.float32)
    v32 = R.rpbh_fp32(x, perm, signs, h).astype(np.float64)
    v64 = R.rpbh_fp64(x.astype(np.float64), perm, signs, h)
    rms = np.sqrt(np.mean(v64 ** 2, axis=1, keepdims=True))
    # well inside the 1e-5 per-element rule used for the GPU comparison
    assert np.max(np.abs(v32 - v64) / np.maximum(np.abs(v64), rms)) < 2e-6


def test_dense32_transform_pair():
    # WUSH review "Core claim": weights take the inverse-transpose of the
    # activation transform, so the product is unchanged
    rng = np.random.default_rng(16)
    nb = 4
    T = rng.standard_normal((nb, 32, 32))
    Tw = np.linalg.inv(T).transpose(0, 2, 1)
    x = rng.standard_normal((3, 32 * nb))
    w = rng.standard_normal((5, 32 * nb))
    lhs = R.dense32_fp64(w, Tw) @ R.dense32_fp64(x, T).T
    np.testing.assert_allclose(lhs, w @ x.T, rtol=1e-9, atol=1e-9)
    # block structure: block b of the output depends on block b of x only
    e = np.zeros(32 * nb)
    e[40] = 1.0
    v = R.dense32_fp64(e, T)
    np.testing.assert_array_equal(v[:32], 0)
    np.testing.assert_allclose(v[32:64], T[1][:, 8])


def test_dense32_weight_transform_is_the_inverse_transpose():
    # WUSH review "Core claim": T_w = T_x^{-T}.  Pinned by the pair identity
    # (T_w w) . (T x) = w . x on the stored bfloat16 matrices, and by
    # T_w^T T = I; the transform family is not orthogonal (diag(s) with s in
    # [0.5, 2]), so an inverse without the transpose fails both.
    import workloads as WL
    wl = WL.make_workload(5, M=3, K=128, Ns=(4,))
    T = WL.bf16_bits_to_f32(wl.t_act_bits).astype(np.float64)
    Tw = R.dense32_weight_transform(wl.t_act_bits)
    for b in range(T.shape[0]):
        np.testing.assert_allclose(Tw[b].T @ T[b], np.eye(32), rtol=0, atol=1e-13)
    x = wl.x_f32.astype(np.float64)
    w = wl.weights[0].astype(np.float64)
    lhs = R.dense32_fp64(w, Tw) @ R.dense32_fp64(x, T).T
    np.testing.assert_allclose(lhs, w @ x.T, rtol=0, atol=1e-12 * np.abs(w @ x.T).max())
    wrong = R.dense32_fp64(w, np.linalg.inv(T)) @ R.dense32_fp64(x, T).T
    assert np.max(np.abs(wrong - w @ x.T)) > 1e-3 * np.abs(w @ x.T).max()


def test_rn32_of_scaled_integers():
    # the integer rounding helper against numpy's float64 -> float32
    # conversion (round to nearest even) wherever the value is exact in float64
    rng = np.random.default_rng(40)
    for _ in range(2000):
        n = int(rng.integers(-(1 << 52), 1 << 52))
        e = int(rng.integers(-170, 60))
        assert R._rn32_scaled_int(n, e) == np.float32(math.ldexp(n, e))
    # ties: 1 + 2^-24 is halfway between 1 and 1 + 2^-23 -> even (1);
    # 1 + 3 2^-24 halfway between 1 + 2^-23 and 1 + 2^-22 -> even (1 + 2^-22)
    assert R._rn32_scaled_int((1 << 24) + 1, -24) == np.float32(1.0)
    assert R._rn32_scaled_int((1 << 24) + 3, -24) == np.float32(1.0 + 2.0 ** -22)
    assert R._rn32_scaled_int(-((1 << 24) + 1), -24) == np.float32(-1.0)


def test_dense32_fp32_is_the_exact_sum_rounded_once():
    # T_b x_b with products 1, 2^-24 and 2^-80: the exact sum lies just above
    # the float32 midpoint 1 + 2^-24, so it rounds up to 1 + 2^-23; a float64
    # sum drops the 2^-80 and the tie then goes to the even neighbour 1
    T = np.zeros((1, 32, 32))
    T[0, 0, :3] = 1.0
    T[0, 1, :2] = 1.0           # 1 + 2^-24 exactly: a true tie -> 1
    T[0, 2, 0] = 0.5            # a plain product
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :3] = [1.0, 2.0 ** -24, 2.0 ** -80]
    v, n_int = R.dense32_fp32(x, T)
    assert v[0, 0] == np.float32(1.0 + 2.0 ** -23)
    assert v[0, 1] == np.float32(1.0)
    assert v[0, 2] == np.float32(0.5)
    assert n_int >= 1
    assert R.dense32_fp64(x, T).astype(np.float32)[0, 0] == np.float32(1.0)   # the float64 shortcut
    # ordinary data: the exponent-span check passes and the float64 sum is used
    import workloads as WL
    wl = WL.make_workload(5, M=64, K=256, Ns=(4,))
    T = WL.bf16_bits_to_f32(wl.t_act_bits)
    v, n_int = R.dense32_fp32(wl.x_f32, T)
    np.testing.assert_array_equal(v, R.dense32_fp64(wl.x_f32, T).astype(np.float32))
