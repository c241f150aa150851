"""Out-of-bounds writes and run-to-run determinism (run with -m gpu).

Every output buffer of the layer's entry points sits between two 4 KiB guard
bands of a canary byte; its interior is filled with different junk before
each of 10 repeats of the same calls.  After every repeat the guard bands must
be intact and every byte the layout defines (rows below M of a tiled operand;
everything else in full) must equal the first repeat's bit for bit.  Sizes
have ragged row counts and span several tiles.  The matrix-core rate probe is
checked for a launch that completes with a rate below the published peak.
"""
import sys

import numpy as np
import pytest

import workloads as WL
from parity import to_dev
from tiling import row_mask, row_mask_mx

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GUARD = 4096
CANARY = 0xA5
REPEATS = 10


@pytest.fixture(scope="module")
def oq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotated_bit_quantized_amd as m
    return m


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Guarded:
    """A device buffer of `nbytes` between two guard bands; `t` is the interior
    as `dtype` of `shape`; `mask` (host bool per interior byte) selects the
    bytes the layout defines."""

    def __init__(self, name, nbytes, dtype=torch.uint8, shape=None, mask=None):
        self.name, self.nbytes, self.mask = name, int(nbytes), mask
        self.buf = torch.full((2 * GUARD + self.nbytes,), CANARY, dtype=torch.uint8, device="cuda")
        t = self.buf[GUARD:GUARD + self.nbytes]
        if dtype != torch.uint8:
            t = t.view(dtype)
        self.t = t.view(shape) if shape is not None else t

    def scramble(self, rep):
        g = torch.Generator().manual_seed(1000 + rep)
        junk = torch.randint(0, 256, (self.nbytes,), dtype=torch.uint8, generator=g)
        self.buf[GUARD:GUARD + self.nbytes].copy_(junk)

    def snapshot(self):
        h = self.buf.cpu().numpy()
        assert (h[:GUARD] == CANARY).all(), f"{self.name}: bytes written before the buffer"
        assert (h[GUARD + self.nbytes:] == CANARY).all(), (
            f"{self.name}: bytes written past the end, first at +"
            f"{int(np.argmax(h[GUARD + self.nbytes:] != CANARY))}")
        inner = h[GUARD:GUARD + self.nbytes]
        return inner[self.mask] if self.mask is not None else inner.copy()


def _repeat(bufs, run, what):
    first = None
    for rep in range(REPEATS):
        for b in bufs:
            b.scramble(rep)
        torch.cuda.synchronize()
        run()
        torch.cuda.synchronize()
        snap = [b.snapshot() for b in bufs]
        if first is None:
            first = snap
            continue
        for b, a0, a in zip(bufs, first, snap):
            assert np.array_equal(a0, a), f"{what}: {b.name} differs between repeat 0 and repeat {rep}"
    say(f"  {what}: {REPEATS} repeats, {len(bufs)} guarded outputs, "
        f"{sum(b.nbytes for b in bufs)} bytes bit-identical")


def _tiled_mask(M, K, planes):
    return np.concatenate([row_mask(M, K)] * planes)


def _mx_scale_mask(M, K):
    Rp = (M + 31) // 32 * 32
    live = np.arange(Rp) < M
    return np.broadcast_to(live[None, :, None], (K // 128, Rp, 4)).reshape(-1)


@pytest.mark.parametrize("cid,M,N", [(2, 300, 640), (3, 77, 384), (4, 161, 256)])
def test_guarded_int_layer(oq, cid, M, N):
    """RPBH rotation + 4/6-bit activation writer (tiled), weight quantizer,
    prepack, tiled FP6 GEMM and the fused layer."""
    say("case guarded int layer", cid, M, N)
    wl = WL.make_workload(cid, M=M, Ns=(N,))
    s, K = wl.spec, wl.K
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), s.block)
    x, W = to_dev(wl.x_bits), to_dev(wl.weights[0])
    afmt = s.afmt | oq.OQ_TILED
    planes = 2 if s.afmt == oq.OQ_A6 else 1
    Np = (N + 31) // 32 * 32

    wc = Guarded("weight codes", N * K // 2, shape=(N, K // 2))
    wsc = Guarded("weight scales", 4 * N * (K // 64), torch.float32, (N, K // 64))
    w1 = Guarded("w1", 4 * N, torch.float32) if s.center else None
    wt = Guarded("tiled weight", oq.oq_tiled_bytes(N, K), mask=_tiled_mask(N, K, 1))
    wst = Guarded("tiled weight scales", 4 * (K // 64) * Np, torch.float32, (K // 64, Np))

    def weights():
        oq.oq_quant_weight(W, rot, oq.OQ_W4, 64, codes=wc.t, scales=wsc.t, w1=None if w1 is None else w1.t,
                           want_w1=s.center)
        oq.oq_prepack_w4(wc.t, wsc.t, N, K, w_tiled=wt.t, w_scale_t=wst.t)

    _repeat([b for b in (wc, wsc, w1, wt, wst) if b is not None], weights, f"c{cid} weight path")
    # the GEMM reads the last repeat's weights, which equal the first's
    codes = Guarded("activation codes", planes * oq.oq_tiled_bytes(M, K), mask=_tiled_mask(M, K, planes))
    scale = Guarded("activation scales", 4 * M, torch.float32)
    mean = Guarded("means", 4 * M, torch.float32) if s.center else None
    y = Guarded("y", 2 * M * N, torch.bfloat16, (M, N))
    yf = Guarded("fused y", 2 * M * N, torch.bfloat16, (M, N))
    ws = Guarded("fused workspace", oq.oq_workspace_bytes(oq.OQ_OP_LINEAR, M, K, N, afmt))
    ws.mask = np.zeros(ws.nbytes, dtype=bool)  # contents are the library's own

    def act_gemm():
        a = oq.oq_quant_act(x, rot, afmt, center=s.center, codes=codes.t, scale=scale.t,
                            mean=None if mean is None else mean.t)
        oq.oq_gemm_w4a4(afmt, a["codes"], a["scale"], wt.t, wst.t, N, 64, mean=a["mean"],
                        w1=None if w1 is None else w1.t, M=M, K=K, y=y.t)
        oq.oq_linear_fused(x, rot, s.center, afmt, wt.t, wst.t, N, 64, w1=None if w1 is None else w1.t,
                           y=yf.t, ws=ws.t)

    _repeat([b for b in (codes, scale, mean, y, yf, ws) if b is not None], act_gemm, f"c{cid} activation path")
    assert torch.equal(y.t.view(torch.int16), yf.t.view(torch.int16)), "fused layer differs from the two-call path"


def test_guarded_w4a8(oq):
    """Row-major 8-bit activations and the W4A8 GEMM (group 128)."""
    M, N = 101, 224
    say("case guarded w4a8", M, N)
    wl = WL.make_workload(1, M=M, Ns=(N,))
    s, K = wl.spec, wl.K
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), s.block)
    x, W = to_dev(wl.x_bits), to_dev(wl.weights[0])
    wq = oq.oq_quant_weight(W, rot, oq.OQ_W4, s.group)
    codes = Guarded("activation codes", M * K, torch.int8, (M, K))
    scale = Guarded("activation scales", 4 * M, torch.float32)
    y = Guarded("y", 2 * M * N, torch.bfloat16, (M, N))

    def run():
        a = oq.oq_quant_act(x, rot, oq.OQ_A8, codes=codes.t, scale=scale.t)
        oq.oq_gemm_w4a8(a["codes"], a["scale"], wq["codes"], wq["scales"], N, s.group, y=y.t)

    _repeat([codes, scale, y], run, "w4a8 path")


def test_guarded_mx_layer(oq):
    """Dense per-32 transforms + tiled MXFP4 writer, weight path, MXFP4 GEMM and
    the fused layer."""
    M, N, K = 130, 288, 1024
    say("case guarded mx layer", M, N, K)
    wl = WL.make_workload(5, M=M, K=K, Ns=(N,))
    rot = oq.Rotation.dense32(to_dev(wl.t_act_bits))
    x, W = to_dev(wl.x_bits), to_dev(wl.weights[0])
    afmt = oq.OQ_MXFP4 | oq.OQ_TILED
    nbw = oq.oq_tiled_mx_bytes(N, K)
    wc = Guarded("weight codes", N * K // 2, shape=(N, K // 2))
    we = Guarded("weight e8m0", N * K // 32, shape=(N, K // 32))
    wt = Guarded("tiled weight", nbw)
    wet = Guarded("tiled weight e8m0", nbw // 16)

    def weights():
        oq.oq_quant_weight(W, rot, oq.OQ_W_MXFP4, 32, codes=wc.t, scales=we.t)
        oq.oq_prepack_mx(wc.t, we.t, N, K, w_tiled=wt.t, w_e8m0_tiled=wet.t)

    _repeat([wc, we, wt, wet], weights, "mx weight path")
    nba = oq.oq_tiled_mx_bytes(M, K)
    codes = Guarded("activation codes", nba, mask=row_mask_mx(M, K))
    e8 = Guarded("activation e8m0", nba // 16, mask=_mx_scale_mask(M, K))
    y = Guarded("y", 2 * M * N, torch.bfloat16, (M, N))
    yf = Guarded("fused y", 2 * M * N, torch.bfloat16, (M, N))
    ws = Guarded("fused workspace", oq.oq_workspace_bytes(oq.OQ_OP_LINEAR, M, K, N, afmt))
    ws.mask = np.zeros(ws.nbytes, dtype=bool)

    def run():
        a = oq.oq_quant_act(x, rot, afmt, codes=codes.t, e8m0=e8.t)
        oq.oq_gemm_w4a4(afmt, a["codes"], a["e8m0"], wt.t, wet.t, N, 32, M=M, K=K, y=y.t)
        oq.oq_linear_fused(x, rot, False, afmt, wt.t, wet.t, N, 32, y=yf.t, ws=ws.t)

    _repeat([codes, e8, y, yf, ws], run, "mx activation path")
    assert torch.equal(y.t.view(torch.int16), yf.t.view(torch.int16)), "fused layer differs from the two-call path"


@pytest.mark.parametrize("kind", ["FP6", "FP4", "FP8", "I8", "BF16", "F16", "FP6_UPDATE"])
def test_probe_rate_below_peak(oq, kind):
    """The probe completes, is deterministic, and its rate stays below the
    published dense peak of its type at the top clock (TFLOP/s or TOPS)."""
    peak = {"FP6": 10100, "FP4": 10100, "FP8": 5000, "I8": 5000, "BF16": 2500, "F16": 2500, "FP6_UPDATE": 10100}[kind]
    k = getattr(oq, "OQ_PROBE_" + kind)
    ops, sink = oq.oq_probe_mfma(k, 200)
    torch.cuda.synchronize()
    first = sink.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    oq.oq_probe_mfma(k, 200, sink)
    e1.record()
    torch.cuda.synchronize()
    rate = ops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    say(f"  probe {kind}: {rate:.0f} of {peak} peak")
    assert torch.equal(first.view(torch.int32), sink.view(torch.int32))
    assert 0.05 * peak < rate < 1.05 * peak
