"""Pins of oracle/gemm.py and oracle/linear.py (CPU only)."""
import numpy as np
import pytest

from oracle import gemm as G
from oracle import linear as L
from oracle import quant as Q
from oracle import rotation as R
import workloads as WL


def _brute_group_acc(qa, qw, group):
    M, K = qa.shape
    N = qw.shape[0]
    out = np.zeros((K // group, M, N), dtype=np.int64)
    for g in range(K // group):
        for t in range(M):
            for o in range(N):
                s = 0
                for k in range(g * group, (g + 1) * group):
                    s += int(qa[t, k]) * int(qw[o, k])
                out[g, t, o] = s
    return out


def test_group_acc_brute_force():
    rng = np.random.default_rng(30)
    qa = rng.integers(-127, 128, size=(3, 128))
    qw = rng.integers(-7, 8, size=(5, 128))
    np.testing.assert_array_equal(G.group_acc(qa, qw, 64), _brute_group_acc(qa, qw, 64))
    assert np.max(np.abs(G.group_acc(qa, qw, 64))) <= 64 * 127 * 7


def test_epilogue_equals_dense_dequantized_product():
    # CentriQ Eq. 5 / Eq. 9 with the quantized operands written out densely:
    # (diag(alpha) Q_a)(Q_w (.) S_w)^T + m w1^T + b
    rng = np.random.default_rng(31)
    M, N, K, g = 4, 6, 256, 64
    qa = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    alpha = rng.uniform(0.1, 2, size=M).astype(np.float32)
    sw = rng.uniform(0.001, 0.01, size=(N, K // g)).astype(np.float32)
    m = rng.standard_normal(M).astype(np.float32)
    w1 = rng.standard_normal(N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    y, S = G.epilogue_int(alpha, G.group_acc(qa, qw, g), sw, m, w1, b)
    Wd = qw * np.repeat(sw.astype(np.float64), g, axis=1)
    dense = (alpha.astype(np.float64)[:, None] * qa) @ Wd.T + np.outer(m, w1) + b
    np.testing.assert_allclose(y, dense.astype(np.float32), rtol=1e-6, atol=1e-6)
    assert np.all(S >= np.abs(dense) - 1e-9)


def test_tolerance_covers_fp32_reorderings():
    rng = np.random.default_rng(32)
    M, N, K, g = 8, 8, 3072, 64
    qa = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    alpha = rng.uniform(0.1, 2, size=M).astype(np.float32)
    sw = rng.uniform(0.001, 0.01, size=(N, K // g)).astype(np.float32)
    acc = G.group_acc(qa, qw, g)
    y, S = G.epilogue_int(alpha, acc, sw)
    # a float32 evaluation in reverse group order must sit inside the tolerance
    F = np.zeros((M, N), dtype=np.float32)
    for gg in reversed(range(K // g)):
        F = (F + sw[:, gg][None, :] * acc[gg].astype(np.float32)).astype(np.float32)
    y32 = (alpha[:, None] * F).astype(np.float32)
    ybf = WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(y32))
    assert np.all(np.abs(ybf.astype(np.float64) - y) <= G.output_tolerance(y, S, K // g))


def test_rank1_restore_is_exact_in_real_arithmetic():
    # CentriQ Eq. 4 and App. C.5: with an identity quantizer the centered,
    # rotated path plus xbar w1 reproduces W x exactly (float64 here)
    rng = np.random.default_rng(33)
    d, h, N = 512, 128, 16
    perm = np.stack([rng.permutation(d)]).astype(np.int32)
    signs = np.where(rng.integers(0, 2, size=(1, d)) == 1, 1, -1).astype(np.int8)
    W = rng.standard_normal((N, d)) * 0.02
    x = rng.standard_normal((5, d)) + rng.normal(0, 3, size=(5, 1))
    m = x.mean(axis=1)
    WR = R.rpbh_fp64(W, perm, signs, h)           # rows w -> R w, i.e. W R^T
    y = R.rpbh_fp64(x - m[:, None], perm, signs, h) @ WR.T + np.outer(m, W.sum(axis=1))
    np.testing.assert_allclose(y, x @ W.T, rtol=0, atol=1e-12)


def test_offset_invariance():
    # CentriQ Eq. 6: y(x + c 1) = y(x) + c w1 for the centered path; inputs
    # chosen so that x + c is exact in bfloat16 and the means differ by c
    rng = np.random.default_rng(34)
    d, h, N, g = 256, 128, 8, 64
    perm = np.stack([rng.permutation(d)]).astype(np.int32)
    signs = np.where(rng.integers(0, 2, size=(1, d)) == 1, 1, -1).astype(np.int8)
    x = np.round(rng.standard_normal((4, d)) * 4) / 4          # multiples of 1/4
    c = 16.0
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    wp = L.prepare_weight_rpbh(W, perm, signs, h, g)
    a0 = L.activations_int(WL.f32_to_bf16_bits(x.astype(np.float32)), perm, signs, h, 4, True)
    a1 = L.activations_int(WL.f32_to_bf16_bits((x + c).astype(np.float32)), perm, signs, h, 4, True)
    np.testing.assert_array_equal(a1["mean"], a0["mean"] + np.float32(c))
    np.testing.assert_array_equal(a1["codes"], a0["codes"])
    y0, S0 = L.linear_int(a0, wp, g)
    y1, S1 = L.linear_int(a1, wp, g)
    np.testing.assert_allclose(y1 - y0, np.outer(np.full(4, c), wp["w1"]), rtol=0, atol=1e-4)


def test_weight_prep_and_forward_small_config():
    wl = WL.make_workload(2, M=8, K=2048, Ns=(64,))
    s = wl.spec
    wp = L.prepare_weight_rpbh(wl.weights[0], wl.perm, wl.signs, s.block, s.group)
    assert wp["packed"].shape == (64, 1024) and wp["scales"].shape == (64, 32)
    np.testing.assert_array_equal(Q.unpack_int4(wp["packed"]), wp["codes"])
    act = L.activations_int(wl.x_bits, wl.perm, wl.signs, s.block, 4, False)
    y, S = L.linear_int(act, wp, s.group)
    # the quantized layer approximates W x: relative error of a W4A4 layer
    ref = wl.x_f32.astype(np.float64) @ wl.weights[0].T.astype(np.float64)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.25


def test_mx_forward_small_config():
    wl = WL.make_workload(5, M=8, K=256, Ns=(32,))
    act = L.activations_mx(wl.x_bits, wl.t_act_bits)
    wp = L.prepare_weight_dense32(wl.weights[0], wl.t_act_bits)
    y, S = L.linear_mx(act, wp)
    ref = wl.x_f32.astype(np.float64) @ wl.weights[0].T.astype(np.float64)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.3
    # the transform pair cancels to float64 rounding
    T = Q.bf16_to_f32(wl.t_act_bits)
    Tw = R.dense32_weight_transform(wl.t_act_bits)
    lhs = R.dense32_fp64(wl.weights[0], Tw) @ R.dense32_fp64(wl.x_f32, T).T
    np.testing.assert_allclose(lhs, ref.T, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_w1_golden_unrotated_row_sums():
    # CentriQ Sec. 4.2 Eq. 4: w_1 = W 1 from the unrotated, unquantized weight
    from conftest import read_golden
    vals = {l.split()[0]: [float(t) for t in l.split()[1:]] for l in read_golden("w1_rowsum.txt")}
    d = 32
    W = np.stack([np.ones(d), np.arange(d) / 8.0]).astype(np.float32)
    perm = np.arange(d, dtype=np.int32)[None]
    signs = np.ones((1, d), dtype=np.int8)
    wp = L.prepare_weight_rpbh(W, perm, signs, 32, 32)
    np.testing.assert_array_equal(wp["w1"], np.array(vals["w1"], dtype=np.float32))
    # the sum of the folded rows is the other (wrong) reading
    np.testing.assert_allclose(wp["rotated"].astype(np.float64).sum(axis=1), vals["rotated_sum"], atol=1e-6)
    assert np.all(np.abs(np.array(vals["rotated_sum"]) - np.array(vals["w1"])) > 1.0)


def test_w1_is_the_correctly_rounded_exact_row_sum():
    # Eq. 4 with the exact row sum rounded once to float32: compared with a
    # rational-arithmetic sum of the unrotated float32 weight, rounded by
    # locating it between its float32 neighbours
    from fractions import Fraction
    rng = np.random.default_rng(35)
    d, h, N = 256, 128, 12
    perm = np.stack([rng.permutation(d)]).astype(np.int32)
    signs = np.where(rng.integers(0, 2, size=(1, d)) == 1, 1, -1).astype(np.int8)
    W = (rng.standard_normal((N, d)) * 0.02 + rng.normal(0, 0.01, size=(N, 1))).astype(np.float32)
    w1 = L.prepare_weight_rpbh(W, perm, signs, h, 64)["w1"]
    for o in range(N):
        exact = sum(Fraction(float(v)) for v in W[o])
        f = w1[o]
        lo = Fraction(float(np.nextafter(f, np.float32(-np.inf))))
        hi = Fraction(float(np.nextafter(f, np.float32(np.inf))))
        here = Fraction(float(f))
        # f is the float32 nearest to the exact sum
        assert abs(exact - here) <= abs(exact - lo) and abs(exact - here) <= abs(exact - hi)
    # a w1 taken from the rotated weight is far off
    wr = L.prepare_weight_rpbh(W, perm, signs, h, 64)["rotated"].astype(np.float64).sum(axis=1)
    assert np.max(np.abs(wr - w1)) > 1e-3
