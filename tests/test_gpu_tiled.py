"""GPU parity of the tiled FP6 path (OQ_TILED): activation writer, weight
prepack, FP6-MFMA GEMM, fused layer; bit-identical to the canonical int8 path
and inside the oracle's tolerance (run with -m gpu)."""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import gemm as OG
from oracle import linear as OL
from oracle import quant as OQ
from parity import check_codes, check_output, to_dev, to_host
from tiling import row_mask, split_a6, tile

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


@pytest.mark.parametrize("M,K,h,rounds,center,afmt", [(37, 1024, 128, 1, False, 4), (70, 3072, 1024, 1, True, 4),
                                                      (33, 1920, 128, 2, False, 6), (5, 256, 32, 1, True, 6),
                                                      # one round, no centring (single row copy): more rows
                                                      # than waves on the chip, a ragged tail, one-slot A6
                                                      (9000, 3072, 1024, 1, False, 4), (77, 1024, 1024, 1, False, 6)])
def test_tiled_activation_writer(oq, M, K, h, rounds, center, afmt):
    say("case tiled act", M, K, h, rounds, center, afmt)
    perm, signs = _meta(K, h, rounds, 11)
    x = np.random.default_rng(M).standard_normal((M, K)) * 2 + (1.0 if center else 0.0)
    xb = WL.f32_to_bf16_bits(x.astype(np.float32))
    rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
    out = oq.oq_quant_act(to_dev(xb), rot, afmt | oq.OQ_TILED, center=center)
    canon = oq.oq_quant_act(to_dev(xb), rot, afmt, center=center)
    torch.cuda.synchronize()
    codes = to_host(canon["codes"])
    codes = OQ.unpack_int4(codes.view(np.uint8)) if afmt == 4 else codes.astype(np.int32)
    ref = OL.activations_int(xb, perm, signs, h, afmt, center)
    check_codes(codes, ref["codes"], ref["flags"], "canonical codes")
    got = to_host(out["codes"])
    plane = oq.oq_tiled_bytes(M, K)
    # rows beyond M are padding the kernel never writes: compare real rows only
    live = row_mask(M, K)

    def real_rows(buf):
        return buf[live]
    if afmt == 4:
        want = tile(codes)
        np.testing.assert_array_equal(real_rows(got[:plane]), real_rows(want))
    else:
        qh, ql = split_a6(codes)
        np.testing.assert_array_equal(real_rows(got[:plane]), real_rows(tile(qh)))
        np.testing.assert_array_equal(real_rows(got[plane:2 * plane]), real_rows(tile(ql)))
    np.testing.assert_array_equal(to_host(out["scale"]), to_host(canon["scale"]))


@pytest.mark.parametrize("N,K", [(96, 256), (300, 1024), (32, 64)])
def test_prepack_layout(oq, N, K):
    say("case prepack", N, K)
    rng = np.random.default_rng(N + K)
    qw = rng.integers(-7, 8, size=(N, K))
    sw = rng.uniform(1e-3, 1e-2, size=(N, K // 64)).astype(np.float32)
    out = oq.oq_prepack_w4(to_dev(OQ.pack_int4(qw)), to_dev(sw), N, K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out["codes"]), tile(qw))
    st = to_host(out["scales"])
    Np = (N + 31) // 32 * 32
    np.testing.assert_array_equal(st[:, :N], sw.T)
    assert np.all(st[:, N:Np] == 0)


GEMM_CASES = [
    # (M, N, K, afmt, rank1, bias)
    (256, 256, 3072, 4, False, False),
    (300, 200, 1024, 4, True, True),
    (64, 512, 1920, 6, False, False),
    (513, 96, 640, 6, True, False),
    (31, 32, 64, 4, False, True),
    (1, 256, 128, 6, False, False),
    # more 256 x 256 tiles than CUs: more than one round of workgroups
    # (the second case has 10 groups per tile, 2 mod 4)
    (4352, 4096, 512, 4, False, False),
    (4352, 4096, 640, 4, True, True),
]


@pytest.mark.parametrize("M,N,K,afmt,rank1,bias", GEMM_CASES)
def test_tiled_gemm(oq, M, N, K, afmt, rank1, bias):
    say("case tiled gemm", M, N, K, afmt, rank1, bias)
    rng = np.random.default_rng(M * 3 + N + K)
    qmax = OQ.qmax_for_bits(afmt)
    qa = rng.integers(-qmax, qmax + 1, size=(M, K))
    qa[0] = qmax
    qa[-1] = -qmax
    qw = rng.integers(-7, 8, size=(N, K))
    alpha = rng.uniform(0.01, 1.0, size=M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, size=(N, K // 64)).astype(np.float32)
    mean = rng.normal(0, 3, size=M).astype(np.float32) if rank1 else None
    w1 = rng.normal(0, 0.5, size=N).astype(np.float32) if rank1 else None
    b = rng.normal(0, 0.1, size=N).astype(np.float32) if bias else None
    kw = dict(mean=None if mean is None else to_dev(mean), w1=None if w1 is None else to_dev(w1),
              bias=None if b is None else to_dev(b))
    wpk = to_dev(OQ.pack_int4(qw))
    wt = oq.oq_prepack_w4(wpk, to_dev(sw), N, K)
    if afmt == 4:
        at = tile(qa)
        y_c = oq.oq_gemm_w4a4(oq.OQ_A4, to_dev(OQ.pack_int4(qa)), to_dev(alpha), wpk, to_dev(sw), N, 64, **kw)
    else:
        qh, ql = split_a6(qa)
        at = np.concatenate([tile(qh), tile(ql)])
        y_c = oq.oq_gemm_w4a8(to_dev(qa.astype(np.int8)), to_dev(alpha), wpk, to_dev(sw), N, 64, **kw)
    y_t = oq.oq_gemm_w4a4(afmt | oq.OQ_TILED, to_dev(at), to_dev(alpha), wt["codes"], wt["scales"], N, 64,
                          M=M, K=K, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y_t.view(torch.int16), y_c.view(torch.int16)), "tiled and canonical GEMMs differ"
    y_ref, S = OG.epilogue_int(alpha, OG.group_acc(qa, qw, 64), sw, mean, w1, b)
    check_output(to_host(y_t), y_ref, S, K // 64, "tiled gemm")


@pytest.mark.parametrize("shape", ["256x256", "256x192", "256x128w8", "256x128", "128x192"])
@pytest.mark.parametrize("M,N,K,rank1,bias", [(300, 520, 1024, True, True), (257, 1000, 512, False, True),
                                              (31, 32, 64, False, False), (600, 3072, 3072, True, False)])
def test_tiled_gemm_shapes(oq, monkeypatch, shape, M, N, K, rank1, bias):
    """Every workgroup shape of the single-plane kernel (8 waves: 256 x 256,
    256 x 192, 256 x 128 outputs; 4 waves: 256 x 128, 128 x 192), forced
    through OQ_FP6_TILE: bit-identical to the canonical GEMM and within the
    bound of the oracle's product."""
    say("case tiled gemm shape", shape, M, N, K, rank1, bias)
    monkeypatch.setenv("OQ_FP6_TILE", shape)
    rng = np.random.default_rng(M + N * 7 + K)
    qa = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    qa[0] = 7
    alpha = rng.uniform(0.01, 1.0, size=M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, size=(N, K // 64)).astype(np.float32)
    mean = rng.normal(0, 3, size=M).astype(np.float32) if rank1 else None
    w1 = rng.normal(0, 0.5, size=N).astype(np.float32) if rank1 else None
    b = rng.normal(0, 0.1, size=N).astype(np.float32) if bias else None
    kw = dict(mean=None if mean is None else to_dev(mean), w1=None if w1 is None else to_dev(w1),
              bias=None if b is None else to_dev(b))
    wpk = to_dev(OQ.pack_int4(qw))
    wt = oq.oq_prepack_w4(wpk, to_dev(sw), N, K)
    y_c = oq.oq_gemm_w4a4(oq.OQ_A4, to_dev(OQ.pack_int4(qa)), to_dev(alpha), wpk, to_dev(sw), N, 64, **kw)
    y_t = oq.oq_gemm_w4a4(oq.OQ_A4 | oq.OQ_TILED, to_dev(tile(qa)), to_dev(alpha), wt["codes"], wt["scales"], N, 64,
                          M=M, K=K, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y_t.view(torch.int16), y_c.view(torch.int16)), "tiled and canonical GEMMs differ"
    y_ref, S = OG.epilogue_int(alpha, OG.group_acc(qa, qw, 64), sw, mean, w1, b)
    check_output(to_host(y_t), y_ref, S, K // 64, "tiled gemm shape " + shape)


@pytest.mark.parametrize("shape", ["256x192", "256x128w8"])
@pytest.mark.parametrize("M,N,K,rank1,bias", [(300, 520, 1024, True, True), (513, 1000, 640, False, True),
                                              (31, 32, 64, False, False), (4352, 4096, 256, False, False)])
def test_tiled_gemm_two_plane_shapes(oq, monkeypatch, shape, M, N, K, rank1, bias):
    """Both workgroup shapes of the two-plane (6-bit activation) kernel,
    forced through OQ_FP6_TILE, including more tiles than CUs: bit-identical
    to the canonical W4A8 GEMM on the same codes and within the bound of the
    oracle's product."""
    say("case tiled gemm two-plane shape", shape, M, N, K, rank1, bias)
    monkeypatch.setenv("OQ_FP6_TILE", shape)
    rng = np.random.default_rng(M * 5 + N + K * 3)
    qa = rng.integers(-31, 32, size=(M, K))
    qa[0] = 31
    qa[-1] = -31
    qw = rng.integers(-7, 8, size=(N, K))
    alpha = rng.uniform(0.01, 1.0, size=M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, size=(N, K // 64)).astype(np.float32)
    mean = rng.normal(0, 3, size=M).astype(np.float32) if rank1 else None
    w1 = rng.normal(0, 0.5, size=N).astype(np.float32) if rank1 else None
    b = rng.normal(0, 0.1, size=N).astype(np.float32) if bias else None
    kw = dict(mean=None if mean is None else to_dev(mean), w1=None if w1 is None else to_dev(w1),
              bias=None if b is None else to_dev(b))
    wpk = to_dev(OQ.pack_int4(qw))
    wt = oq.oq_prepack_w4(wpk, to_dev(sw), N, K)
    qh, ql = split_a6(qa)
    at = np.concatenate([tile(qh), tile(ql)])
    y_c = oq.oq_gemm_w4a8(to_dev(qa.astype(np.int8)), to_dev(alpha), wpk, to_dev(sw), N, 64, **kw)
    y_t = oq.oq_gemm_w4a4(oq.OQ_A6 | oq.OQ_TILED, to_dev(at), to_dev(alpha), wt["codes"], wt["scales"], N, 64,
                          M=M, K=K, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y_t.view(torch.int16), y_c.view(torch.int16)), "two-plane tiled and canonical GEMMs differ"
    y_ref, S = OG.epilogue_int(alpha, OG.group_acc(qa, qw, 64), sw, mean, w1, b)
    check_output(to_host(y_t), y_ref, S, K // 64, "two-plane tiled gemm shape " + shape)


@pytest.mark.parametrize("cid,M,N", [(2, 300, 256), (3, 260, 384), (4, 520, 512)])
def test_tiled_layer(oq, cid, M, N):
    say("case tiled layer", cid, M, N)
    wl = WL.make_workload(cid, M=M, Ns=(N,))
    s = wl.spec
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), s.block)
    wq = oq.oq_quant_weight(to_dev(wl.weights[0]), rot, oq.OQ_W4, s.group, want_w1=s.center)
    wt = oq.oq_prepack_w4(wq["codes"], wq["scales"], N, wl.K)
    x = to_dev(wl.x_bits)
    w1 = wq["w1"] if s.center else None
    y_c = oq.oq_linear_fused(x, rot, s.center, s.afmt, wq["codes"], wq["scales"], N, s.group, w1=w1)
    y_t = oq.oq_linear_fused(x, rot, s.center, s.afmt | oq.OQ_TILED, wt["codes"], wt["scales"], N, s.group, w1=w1)
    act = oq.oq_quant_act(x, rot, s.afmt, center=s.center)
    torch.cuda.synchronize()
    assert torch.equal(y_t.view(torch.int16), y_c.view(torch.int16)), "tiled and canonical layers differ"
    codes = to_host(act["codes"])
    codes = OQ.unpack_int4(codes.view(np.uint8)) if s.afmt == 4 else codes.astype(np.int32)
    aref = OL.activations_int(wl.x_bits, wl.perm, wl.signs, s.block, s.afmt, s.center)
    check_codes(codes, aref["codes"], aref["flags"], "codes")
    a = {"codes": codes, "alpha": to_host(act["scale"]), "mean": None if act["mean"] is None else to_host(act["mean"])}
    wp = {"codes": OQ.unpack_int4(to_host(wq["codes"])), "scales": to_host(wq["scales"]),
          "w1": None if w1 is None else to_host(w1)}
    y_ref, S = OL.linear_int(a, wp, s.group)
    check_output(to_host(y_t), y_ref, S, wl.K // 64, "tiled layer")


@pytest.mark.parametrize("M,K,h,rounds,center,afmt", [(70, 3072, 1024, 1, False, 4), (37, 1024, 128, 1, True, 4),
                                                      (33, 1920, 128, 2, False, 6), (9, 4096, 1024, 2, True, 8),
                                                      (65, 256, 32, 1, False, 8), (3, 32, 32, 0, False, 4)])
def test_percentile_scale(oq, M, K, h, rounds, center, afmt):
    """OQ_SCALE_PCTL (CentriQ Sec. 4.2 "Scale and grid"): scales equal to the
    oracle's, codes bit-exact outside the rounding-boundary exemption, the
    tiled writer bit-identical to the canonical one."""
    say("case percentile", M, K, h, rounds, center, afmt)
    rng = np.random.default_rng(M + K)
    x = rng.standard_normal((M, K)) * rng.uniform(0.5, 4, size=(M, 1)) + (1.5 if center else 0.0)
    x[:, 3] *= 30.0  # an outlier channel the percentile range clips
    xb = WL.f32_to_bf16_bits(x.astype(np.float32))
    if rounds:
        perm, signs = _meta(K, h, rounds, 13)
        rot = oq.Rotation.rpbh(to_dev(perm), to_dev(signs), h)
    else:
        perm = signs = rot = None
    fmt = afmt | oq.OQ_SCALE_PCTL
    canon = oq.oq_quant_act(to_dev(xb), rot, fmt, center=center)
    tiled = oq.oq_quant_act(to_dev(xb), rot, fmt | oq.OQ_TILED, center=center) if afmt in (4, 6) and K % 64 == 0 else None
    torch.cuda.synchronize()
    ref = OL.activations_int(xb, perm, signs, h, afmt, center, pctl=True)
    np.testing.assert_array_equal(to_host(canon["scale"]), ref["alpha"])
    codes = to_host(canon["codes"])
    codes = OQ.unpack_int4(codes.view(np.uint8)) if afmt == 4 else codes.astype(np.int32)
    check_codes(codes, ref["codes"], ref["flags"], "percentile codes")
    qmax = OQ.qmax_for_bits(afmt)
    assert np.any(np.abs(codes) == qmax), "the outlier channel should clip"
    if tiled is not None:
        got = to_host(tiled["codes"])
        plane = oq.oq_tiled_bytes(M, K)
        live = row_mask(M, K)
        if afmt == 4:
            np.testing.assert_array_equal(got[:plane][live], tile(codes)[live])
        else:
            qh, ql = split_a6(codes)
            np.testing.assert_array_equal(got[:plane][live], tile(qh)[live])
            np.testing.assert_array_equal(got[plane:2 * plane][live], tile(ql)[live])
        np.testing.assert_array_equal(to_host(tiled["scale"]), to_host(canon["scale"]))


def test_percentile_layer_fused(oq):
    """oq_linear_fused with the percentile scale equals the separate calls."""
    wl = WL.make_workload(2, M=130, Ns=(256,))
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), 1024)
    wq = oq.oq_quant_weight(to_dev(wl.weights[0]), rot, oq.OQ_W4, 64)
    wt = oq.oq_prepack_w4(wq["codes"], wq["scales"], 256, wl.K)
    fmt = oq.OQ_A4 | oq.OQ_TILED | oq.OQ_SCALE_PCTL
    x = to_dev(wl.x_bits)
    y_f = oq.oq_linear_fused(x, rot, False, fmt, wt["codes"], wt["scales"], 256, 64)
    act = oq.oq_quant_act(x, rot, fmt)
    y_s = oq.oq_gemm_w4a4(oq.OQ_A4 | oq.OQ_TILED, act["codes"], act["scale"], wt["codes"], wt["scales"], 256, 64,
                          M=130, K=wl.K)
    torch.cuda.synchronize()
    assert torch.equal(y_f.view(torch.int16), y_s.view(torch.int16))
    ref = OL.activations_int(wl.x_bits, wl.perm, wl.signs, 1024, 4, False, pctl=True)
    np.testing.assert_array_equal(to_host(act["scale"]), ref["alpha"])
