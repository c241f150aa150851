"""GPU parity of the tiled MXFP4 path (OQ_MXFP4 | OQ_TILED): the dense-transform
activation writer, the weight prepack, the LDS-staged MXFP4 GEMM on tiled
operands and the fused layer; bit-identical to the row-major path and inside
the oracle's tolerance (run with -m gpu)."""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import gemm as OG
from oracle import quant as OQ
from parity import check_output, to_dev, to_host
from tiling import row_mask_mx, tile_mx

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


@pytest.mark.parametrize("M,K", [(70, 256), (3, 4096), (129, 1024), (33, 384)])
def test_tiled_mx_activation_writer(oq, M, K):
    say("case tiled mx act", M, K)
    wl = WL.make_workload(5, M=M, K=K, Ns=(16,))
    rot = oq.Rotation.dense32(to_dev(wl.t_act_bits))
    x = to_dev(wl.x_bits)
    canon = oq.oq_quant_act(x, rot, oq.OQ_MXFP4)
    tiled = oq.oq_quant_act(x, rot, oq.OQ_MXFP4 | oq.OQ_TILED)
    torch.cuda.synchronize()
    want_c, want_s = tile_mx(to_host(canon["codes"]), to_host(canon["e8m0"]))
    got_c, got_s = to_host(tiled["codes"]), to_host(tiled["e8m0"])
    live = row_mask_mx(M, K)
    np.testing.assert_array_equal(got_c[:live.size][live], want_c[live])
    Mp = (M + 31) // 32 * 32
    gs = got_s[:Mp * K // 32].reshape(K // 128, Mp, 4)[:, :M]
    ws = want_s.reshape(K // 128, Mp, 4)[:, :M]
    np.testing.assert_array_equal(gs, ws)


@pytest.mark.parametrize("N,K", [(96, 256), (300, 1024), (32, 128)])
def test_prepack_mx_layout(oq, N, K):
    say("case prepack mx", N, K)
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    e8 = rng.integers(118, 136, size=(N, K // 32)).astype(np.uint8)
    out = oq.oq_prepack_mx(to_dev(codes), to_dev(e8), N, K)
    torch.cuda.synchronize()
    want_c, want_s = tile_mx(codes, e8)
    np.testing.assert_array_equal(to_host(out["codes"])[:want_c.size], want_c)
    np.testing.assert_array_equal(to_host(out["scales"])[:want_s.size], want_s)


@pytest.mark.parametrize("M,N,K,bias", [(130, 96, 256, True), (64, 256, 4096, False), (300, 600, 1152, True),
                                         (1, 40, 128, False), (513, 257, 384, True)])
def test_tiled_mx_gemm(oq, M, N, K, bias):
    say("case tiled mx gemm", M, N, K, bias)
    rng = np.random.default_rng(M * 7 + N + K)
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    ea = rng.integers(118, 136, size=(M, K // 32)).astype(np.uint8)
    ew = rng.integers(118, 136, size=(N, K // 32)).astype(np.uint8)
    b = rng.normal(0, 1, size=N).astype(np.float32) if bias else None
    pa, pw = OQ.pack_nibbles(ca), OQ.pack_nibbles(cw)
    kw = dict(bias=None if b is None else to_dev(b))
    y_c = oq.oq_gemm_w4a4(oq.OQ_MXFP4, to_dev(pa), to_dev(ea), to_dev(pw), to_dev(ew), N, 32, **kw)
    ta, sa = tile_mx(pa, ea)
    wt = oq.oq_prepack_mx(to_dev(pw), to_dev(ew), N, K)
    y_t = oq.oq_gemm_w4a4(oq.OQ_MXFP4 | oq.OQ_TILED, to_dev(ta), to_dev(sa), wt["codes"], wt["scales"], N, 32,
                          M=M, K=K, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y_t.view(torch.int16), y_c.view(torch.int16)), "tiled and row-major MXFP4 GEMMs differ"
    y_ref, S = OG.gemm_mx(OQ.mx_dequant(ca, ea), OQ.mx_dequant(cw, ew), b)
    check_output(to_host(y_t), y_ref, S, K // 32, "tiled mx gemm")


@pytest.mark.parametrize("M,N", [(200, 256), (65, 96)])
def test_tiled_mx_layer(oq, M, N):
    say("case tiled mx layer", M, N)
    wl = WL.make_workload(5, M=M, K=1024, Ns=(N,))
    rot = oq.Rotation.dense32(to_dev(wl.t_act_bits))
    wq = oq.oq_quant_weight(to_dev(wl.weights[0]), rot, oq.OQ_W_MXFP4, 32)
    wt = oq.oq_prepack_mx(wq["codes"], wq["scales"], N, 1024)
    x = to_dev(wl.x_bits)
    y_c = oq.oq_linear_fused(x, rot, False, oq.OQ_MXFP4, wq["codes"], wq["scales"], N, 32)
    y_t = oq.oq_linear_fused(x, rot, False, oq.OQ_MXFP4 | oq.OQ_TILED, wt["codes"], wt["scales"], N, 32)
    act = oq.oq_quant_act(x, rot, oq.OQ_MXFP4 | oq.OQ_TILED)
    y_s = oq.oq_gemm_w4a4(oq.OQ_MXFP4 | oq.OQ_TILED, act["codes"], act["e8m0"], wt["codes"], wt["scales"], N, 32,
                          M=M, K=1024)
    torch.cuda.synchronize()
    assert torch.equal(y_t.view(torch.int16), y_c.view(torch.int16)), "tiled and row-major layers differ"
    assert torch.equal(y_s.view(torch.int16), y_t.view(torch.int16)), "fused and separate tiled calls differ"
