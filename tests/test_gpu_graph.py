"""Graph replay of the layer's launches (run with -m gpu): K1 (rotate +
4-bit tiled codes) and the tiled FP6 GEMM captured in one HIP graph, replayed
several times with eager launches on other inputs and synchronisations in
between; every replay must equal the eager result bit for bit, and the eager
result must match the oracle."""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import linear as OL
from oracle import quant as OQ
from parity import check_codes, to_dev, to_host

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


@pytest.mark.parametrize("center", [False, True])
def test_graph_replay_matches_eager(oq, center):
    say("case graph replay", center)
    M, K, N = 300, 1024, 520
    cid = 4 if center else 2
    wl = WL.make_workload(cid, M=M, K=K, Ns=(N,))
    s = wl.spec
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), s.block)
    wq = oq.oq_quant_weight(to_dev(wl.weights[0]), rot, oq.OQ_W4, 64, want_w1=center)
    wt = oq.oq_prepack_w4(wq["codes"], wq["scales"], N, K)
    fmt = oq.OQ_A4 | oq.OQ_TILED
    rng = np.random.default_rng(5)
    xs = [to_dev(wl.x_bits)] + [to_dev(WL.f32_to_bf16_bits((rng.standard_normal((M, K)) * 2 + 0.5).astype(np.float32)))
                                for _ in range(2)]
    x = xs[0].clone()
    codes = torch.empty(oq.oq_tiled_bytes(M, K), dtype=torch.uint8, device="cuda")
    scale = torch.empty(M, dtype=torch.float32, device="cuda")
    mean = torch.empty(M, dtype=torch.float32, device="cuda") if center else None
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    w1 = wq["w1"] if center else None

    def step():
        oq.oq_quant_act(x, rot, fmt, center=center, codes=codes, scale=scale, mean=mean)
        oq.oq_gemm_w4a4(fmt, codes, scale, wt["codes"], wt["scales"], N, 64, mean=mean, w1=w1, y=y, M=M, K=K)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    # eager reference for each input
    ref = []
    for xi in xs:
        x.copy_(xi)
        step()
        torch.cuda.synchronize()
        ref.append((y.clone(), scale.clone()))
    # the eager step of input 0 against the oracle's codes
    act = oq.oq_quant_act(xs[0], rot, oq.OQ_A4, center=center)
    torch.cuda.synchronize()
    a = OL.activations_int(wl.x_bits, wl.perm, wl.signs, s.block, 4, center)
    check_codes(OQ.unpack_int4(to_host(act["codes"]).view(np.uint8)), a["codes"], a["flags"], "graph-case codes")
    np.testing.assert_array_equal(to_host(act["scale"]), to_host(ref[0][1]))

    for rep in range(6):
        k = rep % len(xs)
        x.copy_(xs[k])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref[k][0].view(torch.int16)), f"replay {rep} differs"
        assert torch.equal(scale, ref[k][1])
        # eager work on another input between replays
        x.copy_(xs[(k + 1) % len(xs)])
        step()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref[(k + 1) % len(xs)][0].view(torch.int16))

