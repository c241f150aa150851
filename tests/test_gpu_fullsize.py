"""Full-size parity of the launches bench.py times (run with -m gpu): every
configuration at its real shape, through the same entry points and operand
layouts, against the oracle on the same seeded inputs.

  * 4096 x 3072 W4A4 (RPBH h = 1024): the tiled 4-bit activation writer
    (every code and scale of the 4096 tokens), both tiled FP6 GEMMs (3072 and
    12288 outputs), every weight code;
  * 4096 x 3072 centred W4A4: the same with the exact mean and the rank-1
    restore in the GEMM epilogue (CentriQ Sec. 4.2 Eq. 4-5);
  * 4096 x 1920 W4A6 (two RPBH rounds, h = 128): the two-plane 6-bit writer
    and the two-plane GEMMs (1920 and 7680 outputs);
  * 8192 x 4096 MXFP4 (dense per-32 transforms): the tiled transform writer
    (every E2M1 code and E8M0 byte) and the tiled MXFP4 GEMM (14336 outputs).

Codes follow the boundary rule (bit-exact except oracle-flagged elements,
counted, below 1e-4); outputs follow the output rule on the GPU's own codes and
scales, on every row where the float64 oracle product takes at most a few
seconds per 1024 rows and on 1024 rows (both ends included) for the widest
linears.  Exempt counts are printed.
"""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import gemm as OG
from oracle import linear as OL
from oracle import quant as OQ
from parity import check_codes, check_output, to_dev, to_host
from tiling import untile, untile_mx

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


_CACHE = {}


def _int_config(oq, cid):
    """K1 in the tiled layout bench.py uses, the weights prepared as bench.py
    prepares them, and both GEMMs; results copied to the host."""
    if cid in _CACHE:
        return _CACHE[cid]
    wl = WL.make_workload(cid)
    s = wl.spec
    say(f"case full size c{cid}: K1 {wl.M}x{wl.K} afmt {s.afmt} tiled, GEMMs {wl.Ns}")
    rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), s.block)
    afmt = s.afmt | oq.OQ_TILED
    act = oq.oq_quant_act(to_dev(wl.x_bits), rot, afmt, center=s.center)
    out = {"wl": wl, "scale": None, "mean": None, "lin": []}
    for W in wl.weights:
        N = W.shape[0]
        wq = oq.oq_quant_weight(to_dev(W), rot, oq.OQ_W4, s.group, want_w1=s.center)
        t = oq.oq_prepack_w4(wq["codes"], wq["scales"], N, wl.K)
        y = oq.oq_gemm_w4a4(afmt, act["codes"], act["scale"], t["codes"], t["scales"], N, 64,
                            mean=act["mean"], w1=wq["w1"], M=wl.M, K=wl.K)
        torch.cuda.synchronize()
        out["lin"].append({"N": N, "y": to_host(y), "wcodes": OQ.unpack_int4(to_host(wq["codes"])),
                           "wscales": to_host(wq["scales"]),
                           "w1": None if wq["w1"] is None else to_host(wq["w1"])})
        del y, t, wq
    buf = to_host(act["codes"])
    plane = oq.oq_tiled_bytes(wl.M, wl.K)
    if s.afmt == oq.OQ_A6:
        out["codes"] = 8 * untile(buf[:plane], wl.M, wl.K) + untile(buf[plane:2 * plane], wl.M, wl.K)
    else:
        out["codes"] = untile(buf[:plane], wl.M, wl.K)
    out["scale"] = to_host(act["scale"])
    if s.center:
        out["mean"] = to_host(act["mean"])
    _CACHE[cid] = out
    return out


def _rows(M, n):
    if n >= M:
        return np.arange(M)
    rng = np.random.default_rng(M + n)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, n - 2, replace=False)]))


def _check_int_outputs(g, lin, rows, group, what):
    """The oracle epilogue (CentriQ Eq. 5 / App. B.2 Eq. 9) of the GPU's own
    codes and scales on the given rows, in chunks of 128 rows."""
    worst = 1.0
    for c0 in range(0, len(rows), 128):
        r = rows[c0:c0 + 128]
        acc = OG.group_acc(g["codes"][r], lin["wcodes"], group)
        mean = None if g["mean"] is None else g["mean"][r]
        y_ref, S = OG.epilogue_int(g["scale"][r], acc, lin["wscales"], mean, lin["w1"] if mean is not None else None)
        worst = min(worst, check_output(lin["y"][r], y_ref, S, lin["wcodes"].shape[1] // group, what))
    return worst


@pytest.mark.parametrize("cid", [2, 4, 3])
def test_full_size_activation_codes(oq, cid):
    g = _int_config(oq, cid)
    wl = g["wl"]
    s = wl.spec
    ref = OL.activations_int(wl.x_bits, wl.perm, wl.signs, s.block, s.afmt, s.center)
    np.testing.assert_array_equal(g["scale"], ref["alpha"])
    if s.center:
        np.testing.assert_array_equal(g["mean"], ref["mean"])
    n = check_codes(g["codes"], ref["codes"], ref["flags"], f"c{cid} activation codes")
    say(f"  c{cid}: {g['codes'].size} codes, {int(ref['flags'].sum())} flagged, {n} differ (all flagged)")


@pytest.mark.parametrize("cid,li,nrows", [(2, 0, 4096), (2, 1, 1024), (4, 0, 4096), (3, 0, 4096), (3, 1, 1024)])
def test_full_size_gemm(oq, cid, li, nrows):
    g = _int_config(oq, cid)
    wl = g["wl"]
    s = wl.spec
    lin = g["lin"][li]
    wref = OL.prepare_weight_rpbh(wl.weights[li], wl.perm, wl.signs, s.block, s.group)
    nw = check_codes(lin["wcodes"], wref["codes"], wref["flags"], f"c{cid} weight codes N={lin['N']}")
    np.testing.assert_array_equal(lin["wscales"], wref["scales"])
    if s.center:
        np.testing.assert_array_equal(lin["w1"], wref["w1"])
    rows = _rows(wl.M, nrows)
    frac = _check_int_outputs(g, lin, rows, s.group, f"c{cid} output N={lin['N']}")
    say(f"  c{cid} N={lin['N']}: weight codes differing (flagged) {nw}; {len(rows)} rows x {lin['N']} outputs "
        f"in tolerance, within 1 bf16 ulp {frac:.6f}")


def test_full_size_mxfp4(oq):
    wl = WL.make_workload(5)
    M, K = wl.M, wl.K
    N = wl.Ns[0]
    say(f"case full size c5: K2 {M}x{K} tiled MXFP4, GEMM N={N}")
    rot = oq.Rotation.dense32(to_dev(wl.t_act_bits))
    afmt = oq.OQ_MXFP4 | oq.OQ_TILED
    act = oq.oq_quant_act(to_dev(wl.x_bits), rot, afmt)
    wq = oq.oq_quant_weight(to_dev(wl.weights[0]), rot, oq.OQ_W_MXFP4, 32)
    t = oq.oq_prepack_mx(wq["codes"], wq["scales"], N, K)
    y = oq.oq_gemm_w4a4(afmt, act["codes"], act["e8m0"], t["codes"], t["scales"], N, 32, M=M, K=K)
    torch.cuda.synchronize()
    cb, eb = untile_mx(to_host(act["codes"]), to_host(act["e8m0"]), M, K)
    acodes = OQ.unpack_nibbles(cb)
    wcodes = OQ.unpack_nibbles(to_host(wq["codes"]))
    wsc = to_host(wq["scales"])
    yg = to_host(y)
    del act, wq, t, y
    aref = OL.activations_mx(wl.x_bits, wl.t_act_bits)
    # E8M0 bytes: equal except blocks whose absmax the oracle flags at a power of two
    eb_bad = (eb != aref["scale_bytes"]) & ~aref["block_flags"]
    assert not eb_bad.any(), f"{int(eb_bad.sum())} unflagged E8M0 mismatches"
    flags = aref["flags"] | np.repeat(aref["block_flags"], 32, axis=1)
    na = check_codes(acodes, aref["codes"], flags, "c5 activation codes")
    wref = OL.prepare_weight_dense32(wl.weights[0], wl.t_act_bits)
    wflags = wref["flags"] | np.repeat(wref["block_flags"], 32, axis=1)
    assert not ((wsc != wref["scale_bytes"]) & ~wref["block_flags"]).any()
    nw = check_codes(wcodes, wref["codes"], wflags, "c5 weight codes")
    say(f"  c5: {acodes.size} activation codes, {int(flags.sum())} flagged, {na} differ; "
        f"{int(aref['exact_int_sums'])} oracle outputs summed in integers; weight codes differing {nw}")
    rows = _rows(M, 1024)
    A = OQ.mx_dequant(acodes[rows], eb[rows])
    Wd = OQ.mx_dequant(wcodes, wsc)
    worst = 1.0
    for c0 in range(0, len(rows), 256):
        y_ref, S = OG.gemm_mx(A[c0:c0 + 256], Wd)
        worst = min(worst, check_output(yg[rows[c0:c0 + 256]], y_ref, S, K // 32, "c5 output"))
    say(f"  c5: {len(rows)} rows x {N} outputs in tolerance, within 1 bf16 ulp {worst:.6f}")
