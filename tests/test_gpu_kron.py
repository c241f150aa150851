"""GPU parity of the factorised Paley x Sylvester rotation (run with -m gpu):
rotated float32 values bit-identical to the oracle's canonical order (and
within 1e-5 of float64), activation codes and scales, weight codes and scales
at the padded width, and the product on those codes, against oracle/kron.py.

Widths cover every Paley order and the padding cases: 1152 = 36 x 32 and
2816 = 44 x 64 and 3072 = 12 x 256 (native), 2240 -> 2304 = 36 x 64 and
5120 -> 5632 = 44 x 128 (padded), 1920 -> 2048 (m = 1, Sylvester stages
across wavefronts), 12288 = 12 x 1024.  The wavefront-per-row kernel takes
m = 1 up to 4096 wide (496 -> 512, 1008 -> 1024, 1920 and 2000 -> 2048,
3504 -> 4096), m = 12 with b = 64, 128, 256 and m = 36, 44 with b = 64
(768, 1504 -> 1536, 2240, 2704 -> 2816, 2816, 3008 -> 3072, 3072); the
other widths run on the workgroup kernel."""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import gemm as OG
from oracle import kron as KR
from oracle import linear as OL
from oracle import quant as OQ
from parity import check_codes, check_output, check_rotated, to_dev, to_host
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


def _x(M, n, center, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, n)) * rng.uniform(0.3, 3, (M, 1)) + (2.0 if center else 0.0)
    x[:, 7] *= 25.0  # an outlier channel
    return WL.f32_to_bf16_bits(x.astype(np.float32))


def _oracle_rot(xb, n, center):
    x32 = OQ.bf16_to_f32(xb)
    mean = None
    if center:
        mean = OQ.token_mean(x32)
        x32 = OQ.center(x32, mean)
    return x32, mean


WIDTHS = [(1152, False), (2816, True), (3072, False), (2240, True), (5120, False), (1920, True), (12288, False),
          (768, True), (1504, False), (2704, True), (3008, True), (1008, False), (496, True), (3504, True),
          (2000, False)]


@pytest.mark.parametrize("n,center", WIDTHS)
def test_kron_rotate(oq, n, center):
    m, b, npad = oq.oq_kron_plan(n)
    say("case kron rotate", n, center, m, b, npad)
    M = 37
    xb = _x(M, n, center, n)
    rot = oq.Rotation.kron(n)
    y, mean = oq.oq_rotate(rot, to_dev(xb), center=center)
    torch.cuda.synchronize()
    x32, mref = _oracle_rot(xb, n, center)
    if center:
        np.testing.assert_array_equal(to_host(mean), mref)
    v32 = KR.rotate_fp32(x32, m, b)
    v64 = KR.rotate_fp64(x32.astype(np.float64), m, b)
    g = to_host(y)
    assert g.shape == (M, npad)
    diff = check_rotated(g, v32, v64, "kron rotated values")
    assert diff == 0, f"{diff} values differ from the canonical float32 order"


@pytest.mark.parametrize("n,center,afmt", [(1152, True, 8), (2240, False, 4), (2816, False, 6), (1920, True, 4),
                                           (3072, False, 4), (1504, True, 4), (768, False, 6), (3008, True, 8),
                                           (2704, True, 6), (3504, False, 4), (496, True, 8)])
def test_kron_quant_act(oq, n, center, afmt):
    m, b, npad = oq.oq_kron_plan(n)
    say("case kron quant", n, center, afmt)
    M = 45
    xb = _x(M, n, center, n + afmt)
    rot = oq.Rotation.kron(n)
    out = oq.oq_quant_act(to_dev(xb), rot, afmt, center=center)
    tiled = oq.oq_quant_act(to_dev(xb), rot, afmt | oq.OQ_TILED, center=center) if afmt in (4, 6) else None
    torch.cuda.synchronize()
    x32, _ = _oracle_rot(xb, n, center)
    v = KR.rotate_fp32(x32, m, b)
    q, alpha, flags = OQ.quant_token_int(v, OQ.qmax_for_bits(afmt))
    codes = to_host(out["codes"])
    codes = OQ.unpack_int4(codes.view(np.uint8)) if afmt == 4 else codes.astype(np.int32)
    assert codes.shape == (M, npad)
    check_codes(codes, q, flags, "kron codes")
    np.testing.assert_array_equal(to_host(out["scale"]), alpha)
    if tiled is not None:
        np.testing.assert_array_equal(to_host(tiled["scale"]), to_host(out["scale"]))
        got = to_host(tiled["codes"])
        plane = oq.oq_tiled_bytes(M, npad)
        live = row_mask(M, npad)
        if afmt == 4:
            np.testing.assert_array_equal(got[:plane][live], tile(codes)[live])
        else:
            qh, ql = split_a6(codes)
            np.testing.assert_array_equal(got[:plane][live], tile(qh)[live])
            np.testing.assert_array_equal(got[plane:2 * plane][live], tile(ql)[live])


@pytest.mark.parametrize("n,N,group", [(1152, 70, 64), (2240, 40, 64), (1920, 33, 128)])
def test_kron_weights(oq, n, N, group):
    m, b, npad = oq.oq_kron_plan(n)
    say("case kron weights", n, N, group)
    W = (np.random.default_rng(n).standard_normal((N, n)) * 0.02).astype(np.float32)
    rot = oq.Rotation.kron(n)
    out = oq.oq_quant_weight(to_dev(W), rot, oq.OQ_W4, group, want_w1=True)
    torch.cuda.synchronize()
    wr = KR.rotate_fp32(W, m, b)
    q, s, flags = OQ.quant_groups_int(wr, group, 7)
    codes = OQ.unpack_int4(to_host(out["codes"]).view(np.uint8))
    check_codes(codes, q, flags, "kron weight codes")
    np.testing.assert_array_equal(to_host(out["scales"]), s)
    np.testing.assert_array_equal(to_host(out["w1"]), OL.row_sums_fp32(W))


@pytest.mark.parametrize("n,N,center", [(2240, 520, True), (1152, 300, False), (2816, 256, True)])
def test_kron_linear(oq, n, N, center):
    """Tiled A4 x W4 at the padded width: y against the oracle's epilogue on
    the GPU's own codes, and against the unquantised product within the
    quantisation error scale."""
    m, b, npad = oq.oq_kron_plan(n)
    say("case kron linear", n, N, center)
    M = 300
    xb = _x(M, n, center, n + N)
    W = (np.random.default_rng(N).standard_normal((N, n)) * 0.02).astype(np.float32)
    rot = oq.Rotation.kron(n)
    wq = oq.oq_quant_weight(to_dev(W), rot, oq.OQ_W4, 64, want_w1=center)
    wt = oq.oq_prepack_w4(wq["codes"], wq["scales"], N, npad)
    act = oq.oq_quant_act(to_dev(xb), rot, oq.OQ_A4 | oq.OQ_TILED, center=center)
    canon = oq.oq_quant_act(to_dev(xb), rot, oq.OQ_A4, center=center)
    y = oq.oq_gemm_w4a4(oq.OQ_A4 | oq.OQ_TILED, act["codes"], act["scale"], wt["codes"], wt["scales"], N, 64,
                        mean=act["mean"], w1=wq["w1"], M=M, K=npad)
    torch.cuda.synchronize()
    qa = OQ.unpack_int4(to_host(canon["codes"]).view(np.uint8))
    qw = OQ.unpack_int4(to_host(wq["codes"]).view(np.uint8))
    acc = OG.group_acc(qa, qw, 64)
    mean = to_host(act["mean"]) if center else None
    w1 = to_host(wq["w1"]) if center else None
    y_ref, S = OG.epilogue_int(to_host(act["scale"]), acc, to_host(wq["scales"]), mean, w1)
    check_output(to_host(y), y_ref, S, npad // 64, "kron linear")
    # the layer is unchanged by the rotation up to quantisation: compare with
    # W x in float64 relative to the output scale
    x64 = OQ.bf16_to_f32(xb).astype(np.float64)
    exact = x64 @ W.astype(np.float64).T
    err = np.abs(to_host(y).astype(np.float64) - exact)
    assert np.median(err) < 0.6 * np.median(np.abs(exact))
