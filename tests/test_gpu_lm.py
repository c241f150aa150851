"""GPU parity of the Lloyd-Max activation path (run with -m gpu): the fused
rotate -> Lloyd-Max writer (canonical level indices and tiled float16 levels),
the float16 weight prepack, and the float16-MFMA GEMM, against the oracle
(oracle/lloyd_max.py) on the same seeded inputs.

Rules:
  * codes: bit-exact except elements the oracle flags within 1e-6 of a
    threshold; rho: bit-exact on every token (the kernel rounds the exact sum
    of squares, recomputing it in integers near a float32 midpoint);
  * tiled levels: equal to the stored level of the canonical code, bit for bit;
  * W16: bit-exact against RN16(s q);
  * outputs: |y - y*| <= ulp_bf16(y*) + (K + 3) 2^-24 S, y* the oracle's
    float64 product of the GPU's own codes and scales rounded once.  The
    float16 products are exact; the matrix cores add them in float32, in
    16-term steps whose rounding is bounded by that of a K-term float32 sum.
"""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import lloyd_max as LM
from oracle import quant as OQ
from oracle import rotation as OR
from parity import check_codes, check_output, to_dev, to_host
from tiling import tile_f16, untile_f16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def oq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotated_bit_quantized_amd as m
    return m


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _meta(K, rounds, seed):
    rng = np.random.default_rng(seed)
    perm = np.stack([rng.permutation(K) for _ in range(rounds)]).astype(np.int32)
    signs = np.where(rng.integers(0, 2, size=(rounds, K)) == 1, 1, -1).astype(np.int8)
    return perm, signs


def _tables(oq, K, bits):
    c16, thr = LM.codebook_tables(K, bits)
    return c16, thr, to_dev(c16.view(np.uint16)), to_dev(thr)


def _oracle_act(xb, perm, signs, h, center, thr):
    x32 = OQ.bf16_to_f32(xb)
    m = None
    if center:
        m = OQ.token_mean(x32)
        x32 = OQ.center(x32, m)
    v = OR.rpbh_fp32(x32, perm, signs, h) if perm is not None else x32
    q, rho = LM.quant_token_lm(v, thr)
    return {"v": v, "codes": q, "rho": rho, "mean": m, "flags": LM.boundary_flags(v, rho, thr)}


def _unpack(codes, bits):
    c = np.asarray(codes).view(np.uint8)
    if bits <= 4:
        out = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
        out[:, 0::2] = c & 0xF
        out[:, 1::2] = c >> 4
        return out
    return c


ACT_CASES = [(37, 1024, 128, 1, False, 4), (70, 3072, 1024, 1, True, 4), (33, 1920, 128, 2, False, 8),
             (9, 4096, 1024, 2, True, 8), (65, 256, 32, 1, False, 2), (3, 32, 32, 0, False, 4),
             (1, 96, 32, 1, True, 6), (40, 512, 512, 1, False, 1)]


@pytest.mark.parametrize("M,K,h,rounds,center,bits", ACT_CASES)
def test_lm_activations(oq, M, K, h, rounds, center, bits):
    say("case lm act", M, K, h, rounds, center, bits)
    rng = np.random.default_rng(M * 7 + K)
    x = rng.standard_normal((M, K)) * rng.uniform(0.2, 5, size=(M, 1)) + (1.5 if center else 0.0)
    x[:, 5] *= 20.0  # an outlier channel
    if M > 2:
        x[1] = 0.0   # an all-zero token: rho is the epsilon floor
    xb = WL.f32_to_bf16_bits(x.astype(np.float32))
    if rounds:
        perm, signs = _meta(K, rounds, 3)
        rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
    else:
        perm = signs = rot = None
    c16, thr, c16_d, thr_d = _tables(oq, K, bits)
    canon = oq.oq_quant_act_lm(to_dev(xb), rot, bits, c16_d, thr_d, tiled=False, center=center)
    tiled = oq.oq_quant_act_lm(to_dev(xb), rot, bits, c16_d, thr_d, tiled=True, center=center)
    torch.cuda.synchronize()
    ref = _oracle_act(xb, perm, signs, h, center, thr)
    rho = to_host(canon["scale"])
    np.testing.assert_array_equal(rho, ref["rho"])
    np.testing.assert_array_equal(to_host(tiled["scale"]), rho)
    if center:
        np.testing.assert_array_equal(to_host(canon["mean"]), ref["mean"])
    codes = _unpack(to_host(canon["codes"]), bits)
    n = check_codes(codes, ref["codes"], ref["flags"], "lm codes")
    if M > 2:
        assert np.all(codes[1] == (1 << (bits - 1)) - 1)  # zero token: the lower central level
    t = untile_f16(to_host(tiled["codes"]).view(np.uint16), M, K)[:M]
    np.testing.assert_array_equal(t, c16.view(np.uint16)[codes])
    say("  flagged mismatches", n)


def test_lm_rho_at_float32_midpoints(oq):
    """Tokens whose RMS sits at or within 2^-48 of the float32 midpoint
    1 + 2^-24 (no rotation, d = 64): rho must be the oracle's RN32(sqrt(RN64(S)
    / d)) of the exact sum S, which the kernel recomputes in integers there.
    The third token's exact S lies above the midpoint's, but RN64(S) is the
    midpoint's, so rho is 1; the fourth rounds up; the rest are scaled copies
    (by powers of two, which keep every square exact) and an ordinary token."""
    say("case lm rho midpoints")
    base = [1.0] * 60 + [2.0, 2.0 ** -9, 2.0 ** -9]
    toks = [base + [c] for c in (2.0 ** -21, 1.5 * 2.0 ** -22, 2.0 ** -21 * (1 + 2.0 ** -7), 1.5 * 2.0 ** -21)]
    toks = toks + [[v * 2.0 ** k for v in t] for t in toks for k in (-20, 17)]
    x = np.array(toks, dtype=np.float32)
    assert np.array_equal(WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(x)), x)  # every coordinate is a bfloat16 value
    x = np.concatenate([x, np.random.default_rng(5).standard_normal((1, 64)).astype(np.float32)])
    xb = WL.f32_to_bf16_bits(x)
    c16, thr, c16_d, thr_d = _tables(oq, 64, 4)
    out = oq.oq_quant_act_lm(to_dev(xb), None, 4, c16_d, thr_d, tiled=False)
    torch.cuda.synchronize()
    ref = _oracle_act(xb, None, None, 0, False, thr)
    rho = to_host(out["scale"])
    np.testing.assert_array_equal(rho, ref["rho"])
    assert rho[0] == np.float32(1.0) and rho[2] == np.float32(1.0)
    assert rho[3] == np.float32(1.0 + 2.0 ** -23)
    check_codes(_unpack(to_host(out["codes"]), 4), ref["codes"], ref["flags"], "lm codes at rho midpoints")


@pytest.mark.parametrize("N,K,group", [(70, 256, 64), (256, 1024, 128), (33, 96, 32)])
def test_prepack_w16(oq, N, K, group):
    say("case prepack w16", N, K, group)
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0, :group] *= 1e-3  # a small group: subnormal-free but many inexact products
    q, s = OQ.quant_groups_int(W, group, 7)[:2]
    w16 = oq.oq_prepack_w16(to_dev(OQ.pack_int4(q)), to_dev(s.astype(np.float32)), N, K, group)
    torch.cuda.synchronize()
    got = untile_f16(to_host(w16).view(np.uint16), N, K)
    ref = LM.weights_f16(q, s, group).view(np.uint16)
    np.testing.assert_array_equal(got[:N], ref)
    assert not got[N:].any()


GEMM_CASES = [(300, 1024, 520, 4, True, True), (257, 512, 256, 8, False, True), (33, 96, 40, 4, False, False),
              (1, 32, 7, 2, True, False), (512, 2048, 768, 8, True, False), (64, 3072, 300, 4, False, True)]


@pytest.mark.parametrize("M,K,N,bits,center,bias", GEMM_CASES)
def test_gemm_lm(oq, M, K, N, bits, center, bias):
    say("case gemm lm", M, K, N, bits, center, bias)
    rng = np.random.default_rng(M + N + K)
    c16, thr, c16_d, _ = _tables(oq, K, bits)
    codes = rng.integers(0, 1 << bits, (M, K)).astype(np.uint8)
    rho = rng.uniform(0.05, 3.0, M).astype(np.float32)
    qw = rng.integers(-7, 8, (N, K))
    group = 32 if K % 64 else 64
    sw = rng.uniform(0.001, 0.02, (N, K // group)).astype(np.float32)
    mean = rng.standard_normal(M).astype(np.float32) if center else None
    w1 = rng.standard_normal(N).astype(np.float32) if center else None
    b = rng.standard_normal(N).astype(np.float32) if bias else None
    w16 = oq.oq_prepack_w16(to_dev(OQ.pack_int4(qw)), to_dev(sw), N, K, group)
    packed = OQ.pack_nibbles(codes) if bits <= 4 else codes
    dev = lambda a: None if a is None else to_dev(a)  # noqa: E731
    y_c = oq.oq_gemm_lm(bits, to_dev(packed), to_dev(rho), w16, N, levels=c16_d, mean=dev(mean), w1=dev(w1),
                        bias=dev(b))
    a_t = to_dev(tile_f16(c16.view(np.uint16)[codes]))
    y_t = oq.oq_gemm_lm(bits, a_t, to_dev(rho), w16, N, tiled=True, mean=dev(mean), w1=dev(w1), bias=dev(b),
                        M=M, K=K)
    torch.cuda.synchronize()
    yc, yt = to_host(y_c), to_host(y_t)
    np.testing.assert_array_equal(yc.view(np.uint32), yt.view(np.uint32))
    y_ref, S = LM.linear_lm(codes, rho, c16, LM.weights_f16(qw, sw, group), mean, w1, b)
    frac = check_output(yc, y_ref, S, K, "lm gemm")
    say("  within 1 bf16 ulp:", frac)


@pytest.mark.parametrize("shape", ["256x384", "256x256", "256x192"])
@pytest.mark.parametrize("M,K,N,bits", [(300, 1024, 520, 4), (257, 512, 1000, 8), (600, 3072, 3072, 4),
                                        (2100, 256, 12288, 4)])
def test_gemm_lm_shapes(oq, monkeypatch, shape, M, K, N, bits):
    """Every workgroup shape of the float16 GEMM, forced through OQ_F16_TILE,
    on ragged sizes and on more tiles than CUs."""
    say("case gemm lm shape", shape, M, K, N, bits)
    monkeypatch.setenv("OQ_F16_TILE", shape)
    rng = np.random.default_rng(M + 5 * N + K)
    c16, thr, c16_d, _ = _tables(oq, K, bits)
    codes = rng.integers(0, 1 << bits, (M, K)).astype(np.uint8)
    rho = rng.uniform(0.05, 3.0, M).astype(np.float32)
    qw = rng.integers(-7, 8, (N, K))
    sw = rng.uniform(0.001, 0.02, (N, K // 64)).astype(np.float32)
    mean = rng.standard_normal(M).astype(np.float32)
    w1 = rng.standard_normal(N).astype(np.float32)
    w16 = oq.oq_prepack_w16(to_dev(OQ.pack_int4(qw)), to_dev(sw), N, K, 64)
    packed = OQ.pack_nibbles(codes) if bits <= 4 else codes
    y = oq.oq_gemm_lm(bits, to_dev(packed), to_dev(rho), w16, N, levels=c16_d, mean=to_dev(mean), w1=to_dev(w1))
    torch.cuda.synchronize()
    y_ref, S = LM.linear_lm(codes, rho, c16, LM.weights_f16(qw, sw, 64), mean, w1, None)
    check_output(to_host(y), y_ref, S, K, "lm gemm shape " + shape)


def test_gemm_lm_empty_and_zero(oq):
    K, N, bits = 64, 40, 4
    c16, thr, c16_d, _ = _tables(oq, K, bits)
    w16 = oq.oq_prepack_w16(to_dev(np.zeros((N, K // 2), np.uint8)), to_dev(np.ones((N, 1), np.float32)), N, K, 64)
    y = oq.oq_gemm_lm(bits, to_dev(np.zeros((0, K // 2), np.uint8)), to_dev(np.zeros(0, np.float32)), w16, N,
                      levels=c16_d)
    torch.cuda.synchronize()
    assert y.shape == (0, N)
    codes = np.full((5, K), 3, np.uint8)
    y = oq.oq_gemm_lm(bits, to_dev(OQ.pack_nibbles(codes)), to_dev(np.ones(5, np.float32)), w16, N, levels=c16_d)
    torch.cuda.synchronize()
    assert not to_host(y).any()  # zero weights


@pytest.mark.parametrize("bits,Ns", [(4, (3072,)), (8, (3072,))])
def test_lm_layer_full_size(oq, bits, Ns):
    """4096 x 3072 workload (the W4A4 DiT linear, RPBH h = 1024): the tiled
    writer and GEMM at full size; codes of sampled tokens against the oracle,
    outputs of sampled tokens against the oracle's product."""
    say("case lm full size", bits, Ns)
    wl = WL.make_workload(2, Ns=Ns)
    M, K = wl.M, wl.K
    c16, thr, c16_d, thr_d = _tables(oq, K, bits)
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), wl.spec.block)
    x = to_dev(wl.x_bits)
    act = oq.oq_quant_act_lm(x, rot, bits, c16_d, thr_d, tiled=True)
    canon = oq.oq_quant_act_lm(x, rot, bits, c16_d, thr_d, tiled=False)
    W = wl.weights[0]
    N = W.shape[0]
    q, s = OQ.quant_groups_int(W, 64, 7)[:2]
    w16 = oq.oq_prepack_w16(to_dev(OQ.pack_int4(q)), to_dev(s.astype(np.float32)), N, K, 64)
    y = oq.oq_gemm_lm(bits, act["codes"], act["scale"], w16, N, tiled=True, M=M, K=K)
    y2 = oq.oq_gemm_lm(bits, canon["codes"], canon["scale"], w16, N, levels=c16_d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(y).view(np.uint32), to_host(y2).view(np.uint32))
    rows = np.sort(np.random.default_rng(bits).choice(M, 48, replace=False))
    ref = _oracle_act(wl.x_bits[rows], wl.perm, wl.signs, wl.spec.block, False, thr)
    codes = _unpack(to_host(canon["codes"])[rows], bits)
    rho = to_host(canon["scale"])[rows]
    np.testing.assert_array_equal(rho, ref["rho"])
    check_codes(codes, ref["codes"], ref["flags"], "lm full-size codes")
    y_ref, S = LM.linear_lm(codes, rho, c16, LM.weights_f16(q, s, 64))
    frac = check_output(to_host(y)[rows], y_ref, S, K, "lm full-size output")
    say("  within 1 bf16 ulp:", frac)
