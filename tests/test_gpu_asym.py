"""GPU parity of the asymmetric-weight path (run with -m gpu): the offline
quantizer (CentriQ Eq. 2, RTN min-max), the activation writer's group sums,
the prepack of q'/2 with sigma and C, and the tiled FP6 GEMM with the
group-sum correction, against the oracle (oracle/asym.py).

Rules: codes bit-exact except oracle-flagged elements (within 1e-6 of a
rounding midpoint); sigma, z, C and the group sums bit-exact; outputs within
ulp_bf16(y*) + (7 G + 3) 2^-24 S, with y* the oracle's float64 product of the
GPU's own activation codes and scales rounded once: every product is exact
in float32 and at most 7 G float32 additions reach each output (6 G correction
products accumulated on the matrix cores, G group updates)."""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import asym as OA
from oracle import linear as OL
from oracle import quant as OQ
from oracle import rotation as OR
from parity import check_codes, check_output, to_dev, to_host
from tiling import row_mask, tile, tile_values

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


def _bits(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _gsum_words(p):
    """Group sums as the GEMM's operand words: bfloat16 8 floor(p / 8) in
    bits 0-15 and p - 8 floor(p / 8) in bits 16-31 (both exact)."""
    p = np.asarray(p, np.int64)
    p1 = (np.floor(p / 8) * 8).astype(np.float32)
    p2 = (p - p1.astype(np.int64)).astype(np.float32)
    return ((p1.view(np.uint32) >> 16) | (p2.view(np.uint32) & 0xFFFF0000)).astype(np.uint32).view(np.int32)


def _gsum_values(words):
    """The group sums a word array holds (the sum of its two bfloat16 pieces)."""
    w = np.asarray(words).view(np.uint32)
    lo = (w << 16).view(np.float32).astype(np.float64)
    hi = (w & 0xFFFF0000).view(np.float32).astype(np.float64)
    return lo + hi


def _weights(N, K, seed):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)) * 0.02 + rng.uniform(-0.01, 0.03, (N, 1))
    W[0, :64] = 0.0  # an all-zero group
    return W.astype(np.float32)


@pytest.mark.parametrize("N,K,h,rounds,group", [(70, 256, 64, 1, 64), (33, 1024, 1024, 1, 128),
                                                (40, 1920, 128, 2, 64), (8, 128, 32, 0, 32)])
def test_quant_weight_asym(oq, N, K, h, rounds, group):
    say("case asym weights", N, K, h, rounds, group)
    W = _weights(N, K, N + K)
    if rounds:
        perm, signs = _meta(K, rounds, 7)
        rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
        wr = OR.rpbh_fp32(W, perm, signs, h)
    else:
        rot, wr = None, W
    out = oq.oq_quant_weight_asym(to_dev(W), rot, group, want_w1=True)
    torch.cuda.synchronize()
    Q, sig, z, flags = OA.quant_groups_asym(wr, group)
    np.testing.assert_array_equal(to_host(out["sigma"]).view(np.uint16), _bits(sig))
    np.testing.assert_array_equal(to_host(out["zero"]).view(np.uint16), _bits(z))
    codes = OQ.unpack_int4(to_host(out["codes"]).view(np.uint8))
    n = check_codes(codes, Q - 8, flags, "asym weight codes")
    np.testing.assert_array_equal(to_host(out["w1"]), OL.row_sums_fp32(W))
    say("  flagged mismatches", n)


@pytest.mark.parametrize("N,K", [(70, 256), (300, 1024)])
def test_prepack_w4_asym(oq, N, K):
    say("case asym prepack", N, K)
    rng = np.random.default_rng(N)
    Q = rng.integers(0, 16, (N, K))
    Q[0, :64] = 0   # q' = -8 everywhere in one group
    Q[1, :64] = 15
    G = K // 64
    sig = OA.bf16_rne(rng.uniform(1e-3, 1e-2, (N, G)).astype(np.float32))
    z = OA.bf16_rne(rng.uniform(-2.0, 17.0, (N, G)).astype(np.float32))
    out = oq.oq_prepack_w4_asym(to_dev(OQ.pack_int4(Q - 8)), to_dev(_bits(sig)), to_dev(_bits(z)), N, K, 64)
    torch.cuda.synchronize()
    Np = (N + 31) // 32 * 32
    want = tile_values((Q - 8) / 2.0)
    got = to_host(out["codes"])[: want.size]
    live = row_mask(N, K)
    np.testing.assert_array_equal(got[live], want[live])
    st = to_host(out["scales"])
    np.testing.assert_array_equal(st[:, :N], sig.T)
    assert not st[:, N:].any()
    pk = to_host(out["corr"]).view(np.uint32)
    assert pk.shape == (G, Np, 2)

    def bf(bits):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    # -C as three bfloat16 pieces: their exact sum is -C
    C = -(bf(pk[..., 0] & 0xFFFF) + bf(pk[..., 0] >> 16) + bf(pk[..., 1] & 0xFFFF))
    np.testing.assert_array_equal(C[:, :N], OA.correction(sig, z).T.astype(np.float64))
    assert not C[:, N:].any()  # padding columns: C = 0 (stored as -0 pieces)
    assert not (pk[..., 1] >> 16).any()


@pytest.mark.parametrize("M,K,h,rounds,center,pctl", [(37, 1024, 128, 1, False, False), (70, 3072, 1024, 1, True, False),
                                                      (9, 256, 64, 1, False, True), (40, 128, 32, 0, False, False)])
def test_act_group_sums(oq, M, K, h, rounds, center, pctl):
    say("case act gsum", M, K, h, rounds, center, pctl)
    rng = np.random.default_rng(M + K)
    x = rng.standard_normal((M, K)) * 2 + (1.0 if center else 0.0)
    xb = WL.f32_to_bf16_bits(x.astype(np.float32))
    if rounds:
        perm, signs = _meta(K, rounds, 5)
        rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
    else:
        perm = signs = rot = None
    fmt = oq.OQ_A4 | oq.OQ_TILED | (oq.OQ_SCALE_PCTL if pctl else 0)
    out = oq.oq_quant_act_gsum(to_dev(xb), rot, fmt, center=center)
    canon = oq.oq_quant_act(to_dev(xb), rot, oq.OQ_A4 | (oq.OQ_SCALE_PCTL if pctl else 0), center=center)
    plain = oq.oq_quant_act(to_dev(xb), rot, fmt, center=center)
    torch.cuda.synchronize()
    codes = OQ.unpack_int4(to_host(canon["codes"]).view(np.uint8))
    ref = OL.activations_int(xb, perm, signs, h, 4, center, pctl=pctl)
    check_codes(codes, ref["codes"], ref["flags"], "codes")
    # the writer with group sums produces the same codes and scales as without
    live = row_mask(M, K)
    np.testing.assert_array_equal(to_host(out["codes"])[live], to_host(plain["codes"])[live])
    np.testing.assert_array_equal(to_host(out["scale"]), to_host(canon["scale"]))
    ref_p = OA.group_sums(codes, 64).T
    got = to_host(out["gsum"])
    np.testing.assert_array_equal(_gsum_values(got), ref_p.astype(np.float64))
    np.testing.assert_array_equal(got.view(np.uint32), _gsum_words(ref_p).view(np.uint32))


GEMM_CASES = [(300, 1024, 520, True, True), (257, 512, 256, False, False), (33, 128, 40, False, True),
              (1, 64, 7, True, False), (512, 3072, 768, False, True)]


@pytest.mark.parametrize("M,K,N,center,bias", GEMM_CASES)
def test_gemm_asym(oq, M, K, N, center, bias):
    say("case gemm asym", M, K, N, center, bias)
    rng = np.random.default_rng(M + N + K)
    G = K // 64
    qa = rng.integers(-7, 8, (M, K))
    qa[0, :64] = 7  # a group sum at its maximum
    alpha = rng.uniform(0.05, 2.0, M).astype(np.float32)
    Q = rng.integers(0, 16, (N, K))
    sig = OA.bf16_rne(rng.uniform(1e-3, 1e-2, (N, G)).astype(np.float32))
    z = OA.bf16_rne(rng.uniform(-1.0, 16.0, (N, G)).astype(np.float32))
    mean = rng.standard_normal(M).astype(np.float32) if center else None
    w1 = rng.standard_normal(N).astype(np.float32) if center else None
    b = rng.standard_normal(N).astype(np.float32) if bias else None
    w = oq.oq_prepack_w4_asym(to_dev(OQ.pack_int4(Q - 8)), to_dev(_bits(sig)), to_dev(_bits(z)), N, K, 64)
    gs = np.ascontiguousarray(_gsum_words(OA.group_sums(qa, 64).T))
    dev = lambda a: None if a is None else to_dev(a)  # noqa: E731
    y = oq.oq_gemm_w4a4_asym(to_dev(tile(qa)), to_dev(alpha), to_dev(gs), w, N, M, K, mean=dev(mean), w1=dev(w1),
                             bias=dev(b))
    torch.cuda.synchronize()
    y_ref, S = OA.linear_asym(alpha, qa, Q, sig, OA.correction(sig, z), 64, mean, w1, b)
    frac = check_output(to_host(y), y_ref, S, 7 * G, "asym gemm")
    say("  within 1 bf16 ulp:", frac)


@pytest.mark.parametrize("shape", ["256x256", "256x192", "256x128w8", "256x128", "128x192"])
@pytest.mark.parametrize("M,K,N", [(300, 1024, 520), (257, 512, 1000), (64, 192, 96)])
def test_gemm_asym_shapes(oq, monkeypatch, shape, M, K, N):
    """Every workgroup shape of the corrected GEMM, forced through OQ_FP6_TILE;
    K = 192 leaves the last pair of groups with one group."""
    say("case gemm asym shape", shape, M, K, N)
    monkeypatch.setenv("OQ_FP6_TILE", shape)
    rng = np.random.default_rng(M + 3 * N + K)
    G = K // 64
    qa = rng.integers(-7, 8, (M, K))
    alpha = rng.uniform(0.05, 2.0, M).astype(np.float32)
    Q = rng.integers(0, 16, (N, K))
    sig = OA.bf16_rne(rng.uniform(1e-3, 1e-2, (N, G)).astype(np.float32))
    z = OA.bf16_rne(rng.uniform(-1.0, 16.0, (N, G)).astype(np.float32))
    b = rng.standard_normal(N).astype(np.float32)
    w = oq.oq_prepack_w4_asym(to_dev(OQ.pack_int4(Q - 8)), to_dev(_bits(sig)), to_dev(_bits(z)), N, K, 64)
    gs = np.ascontiguousarray(_gsum_words(OA.group_sums(qa, 64).T))
    y = oq.oq_gemm_w4a4_asym(to_dev(tile(qa)), to_dev(alpha), to_dev(gs), w, N, M, K, bias=to_dev(b))
    torch.cuda.synchronize()
    y_ref, S = OA.linear_asym(alpha, qa, Q, sig, OA.correction(sig, z), 64, bias=b)
    check_output(to_host(y), y_ref, S, 7 * G, "asym gemm shape " + shape)


def test_asym_layer_full_size(oq):
    """4096 x 3072 -> 3072 (the W4A4 DiT linear, RPBH h = 1024): weights
    quantized asymmetrically on the GPU, activations with group sums, the
    corrected GEMM; sampled tokens against the oracle."""
    say("case asym full size")
    wl = WL.make_workload(2, Ns=(3072,))
    M, K = wl.M, wl.K
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), wl.spec.block)
    W = wl.weights[0]
    N = W.shape[0]
    wq = oq.oq_quant_weight_asym(to_dev(W), rot, 64)
    w = oq.oq_prepack_w4_asym(wq["codes"], wq["sigma"], wq["zero"], N, K, 64)
    act = oq.oq_quant_act_gsum(to_dev(wl.x_bits), rot, oq.OQ_A4 | oq.OQ_TILED)
    canon = oq.oq_quant_act(to_dev(wl.x_bits), rot, oq.OQ_A4)
    y = oq.oq_gemm_w4a4_asym(act["codes"], act["scale"], act["gsum"], w, N, M, K)
    torch.cuda.synchronize()
    qw = OQ.unpack_int4(to_host(wq["codes"]).view(np.uint8)) + 8
    sig = (to_host(wq["sigma"]).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    z = (to_host(wq["zero"]).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    rows = np.sort(np.random.default_rng(11).choice(M, 48, replace=False))
    codes = OQ.unpack_int4(to_host(canon["codes"]).view(np.uint8))[rows]
    ref = OL.activations_int(wl.x_bits[rows], wl.perm, wl.signs, wl.spec.block, 4, False)
    check_codes(codes, ref["codes"], ref["flags"], "full-size codes")
    np.testing.assert_array_equal(_gsum_values(to_host(act["gsum"])[:, rows]),
                                  OA.group_sums(codes, 64).T.astype(np.float64))
    alpha = to_host(act["scale"])[rows]
    y_ref, S = OA.linear_asym(alpha, codes, qw, sig, OA.correction(sig, z), 64)
    frac = check_output(to_host(y)[rows], y_ref, S, 7 * (K // 64), "asym full-size output")
    say("  within 1 bf16 ulp:", frac)
