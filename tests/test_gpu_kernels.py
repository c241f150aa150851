"""GPU parity of every entry point against the oracle at small sizes that span
several tiles and ragged tails (run with -m gpu on an MI355X)."""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import gemm as OG
from oracle import linear as OL
from oracle import quant as OQ
from oracle import rotation as ORot
from parity import check_codes, check_output, check_rotated, to_dev, to_host

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


def _meta(K, h, rounds, seed):
    rng = np.random.default_rng(seed)
    perm = np.stack([rng.permutation(K) for _ in range(rounds)]).astype(np.int32)
    signs = np.where(rng.integers(0, 2, size=(rounds, K)) == 1, 1, -1).astype(np.int8)
    return perm, signs


def _x(M, K, seed, scale=1.0, mean=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * scale + mean
    return WL.f32_to_bf16_bits(x.astype(np.float32))


RPBH_CASES = [
    # (M, K, h, rounds, center)
    (37, 1024, 128, 1, False),
    (19, 3072, 1024, 1, False),
    (23, 1920, 128, 2, False),
    (17, 3072, 1024, 1, True),
    (5, 256, 32, 1, False),
    (9, 512, 64, 2, True),
    (3, 1024, 256, 1, False),
    (4, 2048, 512, 2, False),
    (1, 4096, 1024, 2, True),
    # past the wavefront kernel's 4096: the workgroup kernel, up to the 16384 limit
    (3, 8192, 1024, 2, True),
    (2, 16384, 512, 1, False),
]


@pytest.mark.parametrize("M,K,h,rounds,center", RPBH_CASES)
def test_rotate_rpbh(oq, M, K, h, rounds, center):
    say("case rotate", M, K, h, rounds, center)
    perm, signs = _meta(K, h, rounds, K + h)
    xb = _x(M, K, M * 7 + K, mean=2.0 if center else 0.0)
    rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
    y, mean = oq.oq_rotate(rot, to_dev(xb), center=center)
    torch.cuda.synchronize()
    x32 = OQ.bf16_to_f32(xb)
    if center:
        m = OQ.token_mean(x32)
        np.testing.assert_array_equal(to_host(mean), m)
        x32c = OQ.center(x32, m)
    else:
        x32c = x32
    v32 = ORot.rpbh_fp32(x32c, perm, signs, h)
    v64 = ORot.rpbh_fp64(x32c.astype(np.float64), perm, signs, h)
    ndiff = check_rotated(to_host(y), v32, v64, "rotate")
    assert ndiff == 0, f"{ndiff} elements differ from the canonical float32 order"


@pytest.mark.parametrize("M,K,h,rounds,center", RPBH_CASES[:6])
@pytest.mark.parametrize("afmt", [8, 6, 4])
def test_quant_act_int(oq, M, K, h, rounds, center, afmt):
    say("case quant_act", M, K, h, rounds, center, afmt)
    perm, signs = _meta(K, h, rounds, K + 3 * h)
    xb = _x(M, K, M + K, scale=3.0, mean=-1.5 if center else 0.0)
    rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
    out = oq.oq_quant_act(to_dev(xb), rot, afmt, center=center)
    torch.cuda.synchronize()
    ref = OL.activations_int(xb, perm, signs, h, afmt, center)
    codes = to_host(out["codes"])
    if afmt == 4:
        codes = OQ.unpack_int4(codes.view(np.uint8))
    check_codes(codes.astype(np.int32), ref["codes"], ref["flags"], "act codes")
    np.testing.assert_array_equal(to_host(out["scale"]), ref["alpha"])
    if center:
        np.testing.assert_array_equal(to_host(out["mean"]), ref["mean"])


@pytest.mark.parametrize("M,K,h,rounds,center,afmt", [(5, 8192, 1024, 2, True, 4), (3, 16384, 256, 1, False, 8),
                                                      (4, 6144, 1024, 1, False, 6)])
def test_quant_act_widest(oq, M, K, h, rounds, center, afmt):
    """Widths above 4096 (the workgroup kernel) up to the 16384 limit."""
    say("case quant_act widest", M, K, h, rounds, center, afmt)
    perm, signs = _meta(K, h, rounds, K + h)
    xb = _x(M, K, M + 3 * K, scale=2.0, mean=1.0 if center else 0.0)
    rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
    out = oq.oq_quant_act(to_dev(xb), rot, afmt, center=center)
    torch.cuda.synchronize()
    ref = OL.activations_int(xb, perm, signs, h, afmt, center)
    codes = to_host(out["codes"])
    if afmt == 4:
        codes = OQ.unpack_int4(codes.view(np.uint8))
    check_codes(codes.astype(np.int32), ref["codes"], ref["flags"], "act codes")
    np.testing.assert_array_equal(to_host(out["scale"]), ref["alpha"])
    if center:
        np.testing.assert_array_equal(to_host(out["mean"]), ref["mean"])


def test_quant_act_no_rotation_and_edge_rows(oq):
    say("case quant_act edge rows")
    K = 256
    x = np.random.default_rng(5).standard_normal((6, K)).astype(np.float32)
    x[0] = 0.0                       # all-zero token: eps floor, codes 0
    x[1] = 3.25                      # constant token
    x[2] = 0.0
    x[2, 17] = -40.0                 # a single spike saturates to -qmax
    x[3] = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    xb = WL.f32_to_bf16_bits(x)
    for afmt in (8, 4):
        for center in (False, True):
            out = oq.oq_quant_act(to_dev(xb), None, afmt, center=center)
            torch.cuda.synchronize()
            x32 = OQ.bf16_to_f32(xb)
            m = None
            if center:
                m = OQ.token_mean(x32)
                x32 = OQ.center(x32, m)
            q, alpha, flags = OQ.quant_token_int(x32, OQ.qmax_for_bits(afmt))
            codes = to_host(out["codes"])
            if afmt == 4:
                codes = OQ.unpack_int4(codes.view(np.uint8))
            check_codes(codes.astype(np.int32), q, flags, "edge codes")
            np.testing.assert_array_equal(to_host(out["scale"]), alpha)
            assert np.all(codes[0] == 0)
    # identity metadata reduces to the plain block Sylvester transform
    perm = np.arange(K, dtype=np.int32)[None]
    signs = np.ones((1, K), dtype=np.int8)
    rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), 64)
    y, _ = oq.oq_rotate(rot, to_dev(xb))
    torch.cuda.synchronize()
    from oracle.hadamard import fwht_fp32_canonical
    np.testing.assert_array_equal(to_host(y), fwht_fp32_canonical(OQ.bf16_to_f32(xb), 64))


def test_empty_batch_is_noop(oq):
    x = torch.empty((0, 1024), dtype=torch.int16, device="cuda")
    perm, signs = _meta(1024, 128, 1, 1)
    rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), 128)
    out = oq.oq_quant_act(x, rot, 8)
    y, _ = oq.oq_rotate(rot, x)
    torch.cuda.synchronize()
    assert out["codes"].shape == (0, 1024) and y.shape == (0, 1024)


@pytest.mark.parametrize("N,K,h,rounds,group", [(40, 1024, 128, 1, 128), (33, 3072, 1024, 1, 64),
                                                  (16, 1920, 128, 2, 64), (8, 512, 32, 1, 32)])
def test_quant_weight_rpbh(oq, N, K, h, rounds, group):
    say("case quant_weight", N, K, h, rounds, group)
    perm, signs = _meta(K, h, rounds, 99)
    W = (np.random.default_rng(N).standard_normal((N, K)) * 0.02).astype(np.float32)
    rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
    out = oq.oq_quant_weight(to_dev(W), rot, oq.OQ_W4, group, want_w1=True)
    torch.cuda.synchronize()
    ref = OL.prepare_weight_rpbh(W, perm, signs, h, group)
    codes = OQ.unpack_int4(to_host(out["codes"]))
    check_codes(codes, ref["codes"], ref["flags"], "weight codes")
    np.testing.assert_array_equal(to_host(out["scales"]), ref["scales"])
    w1 = to_host(out["w1"])
    assert np.all(np.abs(w1 - ref["w1"]) <= np.spacing(np.abs(ref["w1"])))


@pytest.mark.parametrize("M,K", [(70, 256), (3, 4096), (129, 1024)])
def test_dense32_rotate_and_mx(oq, M, K):
    say("case dense32", M, K)
    wl = WL.make_workload(5, M=M, K=K, Ns=(16,))
    T = to_dev(wl.t_act_bits)
    rot = oq.Rotation.dense32(T)
    y, _ = oq.oq_rotate(rot, to_dev(wl.x_bits))
    out = oq.oq_quant_act(to_dev(wl.x_bits), rot, oq.OQ_MXFP4)
    torch.cuda.synchronize()
    ref = OL.activations_mx(wl.x_bits, wl.t_act_bits)
    v64 = ORot.dense32_fp64(wl.x_f32, OQ.bf16_to_f32(wl.t_act_bits))
    ndiff = check_rotated(to_host(y), ref["rotated"], v64, "dense32")
    assert ndiff == 0
    np.testing.assert_array_equal(to_host(out["e8m0"]), ref["scale_bytes"])
    codes = OQ.unpack_nibbles(to_host(out["codes"]))
    check_codes(codes, ref["codes"], ref["flags"], "mx codes")


def _boundary_case(M, K, seed):
    """Signed-permutation transforms and inputs on E2M1 rounding midpoints,
    grid points and powers of two, so that products are exact, many elements
    sit exactly on a tie and many block maxima are powers of two (exponent
    boundaries): the cases where a float32-accumulated value cannot decide
    the code and the exact recompute must."""
    rng = np.random.default_rng(seed)
    nb = K // 32
    T = np.zeros((nb, 32, 32), dtype=np.float32)
    for b in range(nb):
        T[b, np.arange(32), rng.permutation(32)] = rng.choice([-1.0, 1.0], size=32)
    mags = np.array([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0, 8.0],
                    dtype=np.float32)
    x = rng.choice(mags, size=(M, K)) * rng.choice([-1.0, 1.0], size=(M, K))
    x = x * np.repeat(np.exp2(rng.integers(-20, 20, size=(M, nb))), 32, axis=1)
    return WL.f32_to_bf16_bits(x.astype(np.float32)), WL.f32_to_bf16_bits(T)


@pytest.mark.parametrize("M,K", [(97, 256), (64, 4096)])
def test_dense32_mx_boundaries_exact(oq, M, K):
    say("case dense32 mx boundaries", M, K)
    xb, tb = _boundary_case(M, K, M + K)
    rot = oq.Rotation.dense32(to_dev(tb))
    ref = OL.activations_mx(xb, tb)
    for afmt in (oq.OQ_MXFP4, oq.OQ_MXFP4 | oq.OQ_TILED):
        out = oq.oq_quant_act(to_dev(xb), rot, afmt)
        torch.cuda.synchronize()
        if afmt & oq.OQ_TILED:
            Mp = (M + 31) // 32 * 32
            sb = to_host(out["e8m0"])[:Mp * K // 32].reshape(K // 128, Mp, 4)[:, :M].transpose(1, 0, 2)
            np.testing.assert_array_equal(sb.reshape(M, K // 32), ref["scale_bytes"])
            continue
        np.testing.assert_array_equal(to_host(out["e8m0"]), ref["scale_bytes"])
        np.testing.assert_array_equal(OQ.unpack_nibbles(to_host(out["codes"])), ref["codes"])


def test_dense32_mx_every_element(oq):
    """1536 tokens x 4096 (6.3M elements, config-5 width): every code and
    scale byte against the oracle."""
    M, K = 1536, 4096
    say("case dense32 mx every element", M, K)
    wl = WL.make_workload(5, M=M, K=K, Ns=(16,))
    rot = oq.Rotation.dense32(to_dev(wl.t_act_bits))
    out = oq.oq_quant_act(to_dev(wl.x_bits), rot, oq.OQ_MXFP4)
    torch.cuda.synchronize()
    ref = OL.activations_mx(wl.x_bits, wl.t_act_bits)
    np.testing.assert_array_equal(to_host(out["e8m0"]), ref["scale_bytes"])
    n = check_codes(OQ.unpack_nibbles(to_host(out["codes"])), ref["codes"], ref["flags"], "mx codes")
    say(f"  codes differing on exempt elements: {n}")


def test_weight_dense32(oq):
    say("case weight dense32")
    wl = WL.make_workload(5, M=4, K=512, Ns=(48,))
    rot = oq.Rotation.dense32(to_dev(wl.t_act_bits))
    out = oq.oq_quant_weight(to_dev(wl.weights[0]), rot, oq.OQ_W_MXFP4, 32)
    torch.cuda.synchronize()
    ref = OL.prepare_weight_dense32(wl.weights[0], wl.t_act_bits)
    sb = to_host(out["scales"])
    ok_blocks = ~ref["block_flags"]
    assert np.all((sb == ref["scale_bytes"]) | ~ok_blocks)
    codes = OQ.unpack_nibbles(to_host(out["codes"]))
    flags = ref["flags"] | np.repeat(ref["block_flags"], 32, axis=1)
    check_codes(codes, ref["codes"], flags, "mx weight codes")


GEMM_CASES = [
    # (M, N, K, group, afmt, rank1, bias)
    (130, 136, 1024, 128, 8, False, False),
    (64, 256, 3072, 64, 4, False, True),
    (257, 96, 1920, 64, 6, False, False),
    (100, 160, 3072, 64, 4, True, True),
    (1, 32, 256, 32, 8, True, False),
    (33, 64, 512, 128, 4, False, False),
]


def _rand_codes(rng, M, K, qmax):
    return rng.integers(-qmax, qmax + 1, size=(M, K)).astype(np.int32)


@pytest.mark.parametrize("M,N,K,group,afmt,rank1,bias", GEMM_CASES)
def test_gemm_int(oq, M, N, K, group, afmt, rank1, bias):
    say("case gemm_int", M, N, K, group, afmt, rank1, bias)
    rng = np.random.default_rng(M * N + K)
    qmax = OQ.qmax_for_bits(afmt)
    qa = _rand_codes(rng, M, K, qmax)
    qa[0, :] = qmax                                     # saturated row
    qw = _rand_codes(rng, N, K, 7)
    alpha = rng.uniform(0.01, 1.0, size=M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, size=(N, K // group)).astype(np.float32)
    mean = rng.normal(0, 3, size=M).astype(np.float32) if rank1 else None
    w1 = rng.normal(0, 0.5, size=N).astype(np.float32) if rank1 else None
    b = rng.normal(0, 0.1, size=N).astype(np.float32) if bias else None
    wpk = OQ.pack_int4(qw)
    args = dict(mean=None if mean is None else to_dev(mean), w1=None if w1 is None else to_dev(w1),
                bias=None if b is None else to_dev(b))
    if afmt == 4:
        y = oq.oq_gemm_w4a4(oq.OQ_A4, to_dev(OQ.pack_int4(qa)), to_dev(alpha), to_dev(wpk), to_dev(sw), N, group, **args)
    else:
        y = oq.oq_gemm_w4a8(to_dev(qa.astype(np.int8)), to_dev(alpha), to_dev(wpk), to_dev(sw), N, group, **args)
    torch.cuda.synchronize()
    acc = OG.group_acc(qa, qw, group)
    y_ref, S = OG.epilogue_int(alpha, acc, sw, mean, w1, b)
    frac = check_output(to_host(y), y_ref, S, K // group, "gemm_int")
    say("  within 1 bf16 ulp:", frac)


def _small_product(M, N, K):
    """The library's routing of W4A8 products: fewer 128 x 128 tiles than 128
    and K <= 4096 run the 32 x 32 tile kernel (4 waves of 16 x 16)."""
    return K <= 4096 and -(-N // 128) * -(-M // 128) < 128


def _w4a8_case(M, N, K, group, qmax, rank1, bias, seed):
    rng = np.random.default_rng(seed)
    qa = _rand_codes(rng, M, K, qmax)
    qa[0, :] = qmax
    qw = _rand_codes(rng, N, K, 7)
    alpha = rng.uniform(0.01, 1.0, size=M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, size=(N, K // group)).astype(np.float32)
    mean = rng.normal(0, 3, size=M).astype(np.float32) if rank1 else None
    w1 = rng.normal(0, 0.5, size=N).astype(np.float32) if rank1 else None
    b = rng.normal(0, 0.1, size=N).astype(np.float32) if bias else None
    args = dict(mean=None if mean is None else to_dev(mean), w1=None if w1 is None else to_dev(w1),
                bias=None if b is None else to_dev(b))
    dev = (to_dev(qa.astype(np.int8)), to_dev(alpha), to_dev(OQ.pack_int4(qw)), to_dev(sw))
    acc = OG.group_acc(qa, qw, group)
    y_ref, S = OG.epilogue_int(alpha, acc, sw, mean, w1, b)
    return dev, args, y_ref, S


@pytest.mark.parametrize("M,N,K,group,qmax,rank1,bias", [(256, 1024, 1024, 128, 127, False, False),
                                                          (77, 200, 512, 64, 127, True, True),
                                                          (1, 32, 256, 32, 31, True, False),
                                                          (130, 136, 1024, 128, 127, False, True),
                                                          (64, 96, 192, 32, 127, False, False),
                                                          (64, 96, 8192, 128, 127, True, True)])
def test_gemm_w4a8_split(oq, M, N, K, group, qmax, rank1, bias, monkeypatch):
    """The W4A8 product split across K through the optional scratch (small
    products with K <= 4096 reach it with OQ_INT_SMALL=0, larger K by
    default): against the oracle under the output rule with the extra
    float32 additions of the partial sums counted, repeatable bit for bit,
    and the one-pass call on the same inputs within the same rule."""
    say("case gemm_w4a8 split", M, N, K, group, qmax, rank1, bias)
    if _small_product(M, N, K):
        monkeypatch.setenv("OQ_INT_SMALL", "0")
    (A, AL, W, SW), args, y_ref, S = _w4a8_case(M, N, K, group, qmax, rank1, bias, 7 * M + N + K)
    nbytes = oq.oq_workspace_bytes(oq.OQ_OP_GEMM_W4A8, M, K, N, 0)
    tiles = -(-N // 128) * -(-M // 128)
    splits = 1 if tiles >= 128 else min(-(-256 // tiles), K // group)
    assert (nbytes > 0) == (splits > 1)
    ws = torch.zeros(max(16, nbytes), dtype=torch.uint8, device="cuda")
    y1 = oq.oq_gemm_w4a8(A, AL, W, SW, N, group, ws=ws, **args)
    y2 = oq.oq_gemm_w4a8(A, AL, W, SW, N, group, ws=ws, **args)
    y0 = oq.oq_gemm_w4a8(A, AL, W, SW, N, group, **args)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "split product not repeatable"
    frac = check_output(to_host(y1), y_ref, S, K // group + splits, "gemm_w4a8 split")
    check_output(to_host(y0), y_ref, S, K // group, "gemm_w4a8 one pass")
    say(f"  {splits} splits, within 1 bf16 ulp: {frac}")


@pytest.mark.parametrize("M,N,K,group,qmax,rank1,bias", [(256, 1024, 1024, 128, 127, False, False),
                                                          (45, 70, 1088, 64, 127, True, True),
                                                          (1, 32, 256, 32, 31, True, False),
                                                          (97, 33, 2048, 1024, 127, False, True),
                                                          (40, 300, 4096, 32, 127, True, False),
                                                          (512, 200, 1920, 64, 31, False, True),
                                                          (7, 1000, 64, 32, 127, False, False),
                                                          (64, 64, 4096, 2048, 127, True, True)])
def test_gemm_w4a8_small(oq, M, N, K, group, qmax, rank1, bias, monkeypatch):
    """Small W4A8 products on the 32 x 32 tile kernel (chunks of 1024 k, a
    ragged last chunk, groups of 32 to 2048, the largest spanning two
    chunks, ragged M and N): against the oracle under the output rule,
    and bit-identical to the one-pass kernel (OQ_INT_SMALL=0, no scratch),
    whose fold and epilogue arithmetic it repeats."""
    say("case gemm_w4a8 small", M, N, K, group, qmax, rank1, bias)
    assert _small_product(M, N, K)
    (A, AL, W, SW), args, y_ref, S = _w4a8_case(M, N, K, group, qmax, rank1, bias, 11 * M + N + K)
    assert oq.oq_workspace_bytes(oq.OQ_OP_GEMM_W4A8, M, K, N, 0) == 0
    ys = oq.oq_gemm_w4a8(A, AL, W, SW, N, group, **args)
    ys2 = oq.oq_gemm_w4a8(A, AL, W, SW, N, group, **args)
    monkeypatch.setenv("OQ_INT_SMALL", "0")
    y0 = oq.oq_gemm_w4a8(A, AL, W, SW, N, group, **args)
    torch.cuda.synchronize()
    assert torch.equal(ys.view(torch.int16), ys2.view(torch.int16)), "small product not repeatable"
    frac = check_output(to_host(ys), y_ref, S, K // group, "gemm_w4a8 small")
    assert torch.equal(ys.view(torch.int16), y0.view(torch.int16)), "small and one-pass kernels differ"
    say(f"  within 1 bf16 ulp: {frac}")


@pytest.mark.parametrize("M,N,K,bias", [(130, 96, 256, True), (64, 256, 4096, True), (7, 32, 64, True),
                                         (300, 600, 1152, True), (1, 40, 128, False), (513, 257, 384, False),
                                         (260, 300, 192, True)])
def test_gemm_mx(oq, M, N, K, bias):
    # K % 128 == 0 runs the LDS-staged kernel (several stages, ragged M and N
    # tiles, a single stage at K = 128), other K the direct-load kernel
    say("case gemm_mx", M, N, K, bias)
    rng = np.random.default_rng(M + N + K)
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    ea = rng.integers(118, 136, size=(M, K // 32)).astype(np.uint8)
    ew = rng.integers(118, 136, size=(N, K // 32)).astype(np.uint8)
    b = rng.normal(0, 1, size=N).astype(np.float32) if bias else None
    y = oq.oq_gemm_w4a4(oq.OQ_MXFP4, to_dev(OQ.pack_nibbles(ca)), to_dev(ea), to_dev(OQ.pack_nibbles(cw)),
                        to_dev(ew), N, 32, bias=None if b is None else to_dev(b))
    torch.cuda.synchronize()
    y_ref, S = OG.gemm_mx(OQ.mx_dequant(ca, ea), OQ.mx_dequant(cw, ew), b)
    check_output(to_host(y), y_ref, S, K // 32, "gemm_mx")


def test_determinism(oq):
    say("case determinism")
    wl = WL.make_workload(2, M=300, K=3072, Ns=(256,))
    s = wl.spec
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), s.block)
    wq = oq.oq_quant_weight(to_dev(wl.weights[0]), rot, oq.OQ_W4, s.group)
    x = to_dev(wl.x_bits)
    ys = [oq.oq_linear_fused(x, rot, False, oq.OQ_A4, wq["codes"], wq["scales"], 256, s.group) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
