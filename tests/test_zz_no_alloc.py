"""The entry point that allocates nothing (run with -m gpu): its output equals
oq_linear_fused's bit for bit, through the C ABI, on two calls in a row (the
second smaller, so the scratch still holds the first call's larger codes),
for the tiled 4-bit, the 6-bit and the tiled MXFP4 layers; a layer whose
workspace exceeds the static scratch is refused before any launch."""
import sys

import numpy as np
import pytest

import workloads as WL
from parity import to_dev, to_host

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


def _layer(oq, cid, M, N):
    wl = WL.make_workload(cid, M=M, Ns=(N,))
    s = wl.spec
    W = to_dev(wl.weights[0])
    if s.rot == "rpbh":
        rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), s.block)
        wq = oq.oq_quant_weight(W, rot, oq.OQ_W4, s.group, want_w1=s.center)
        t = oq.oq_prepack_w4(wq["codes"], wq["scales"], N, wl.K)
        return wl, rot, s.afmt | oq.OQ_TILED, t["codes"], t["scales"], wq["w1"], 64
    rot = oq.Rotation.dense32(to_dev(wl.t_act_bits))
    wq = oq.oq_quant_weight(W, rot, oq.OQ_W_MXFP4, 32)
    t = oq.oq_prepack_mx(wq["codes"], wq["scales"], N, wl.K)
    return wl, rot, oq.OQ_MXFP4 | oq.OQ_TILED, t["codes"], t["scales"], None, 32


@pytest.mark.parametrize("cid,M1,M2,N", [(2, 4096, 1000, 3072), (4, 2048, 77, 512), (3, 1536, 33, 640),
                                         (5, 4096, 300, 1024)])
def test_noalloc_equals_fused(oq, cid, M1, M2, N):
    say("case noalloc", cid, M1, M2, N)
    for M in (M1, M2):
        wl, rot, afmt, w, ws, w1, group = _layer(oq, cid, M, N)
        x = to_dev(wl.x_bits)
        y_ref = oq.oq_linear_fused(x, rot, wl.spec.center, afmt, w, ws, N, group, w1=w1)
        torch.cuda.synchronize()
        y = oq.oq_linear_fused_noalloc(x, rot, wl.spec.center, afmt, w, ws, N, group, w1=w1)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"noalloc differs at M={M}"
        say(f"  M={M}: {M * N} outputs equal")


def test_noalloc_refuses_beyond_scratch(oq):
    say("case noalloc too large")
    K, N = 4096, 256
    M = 2 * oq.OQ_NOALLOC_SCRATCH_BYTES // (K // 2)   # INT4 codes alone exceed the scratch
    assert oq.oq_workspace_bytes(oq.OQ_OP_LINEAR, M, K, N, oq.OQ_A4) > oq.OQ_NOALLOC_SCRATCH_BYTES
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((N, K // 64), dtype=torch.float32, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(oq.OQError) as e:
        oq.oq_linear_fused_noalloc(x, None, False, oq.OQ_A4, w, sc, N, 64, y=y)
    assert e.value.code == oq.OQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())   # nothing was launched
