"""GPU parity of the whole layer for the five configurations: reduced sizes
compared element by element, and the full sizes in the launch configuration
the benchmark times, compared on sampled rows (run with -m gpu)."""
import sys

import numpy as np
import pytest

import workloads as WL
from oracle import gemm as OG
from oracle import linear as OL
from oracle import quant as OQ
from parity import check_codes, check_output, to_dev, to_host

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


def _gpu_layer(oq, wl, n_index=0, rows=None):
    """Runs weight prep, activation quantization, the GEMM and the fused call
    on the GPU; returns host copies."""
    s = wl.spec
    W = wl.weights[n_index]
    N = W.shape[0]
    x = to_dev(wl.x_bits)
    if s.rot == "rpbh":
        rot = oq.Rotation.rpbh(to_dev(wl.perm), to_dev(wl.signs), s.block)
        wq = oq.oq_quant_weight(to_dev(W), rot, oq.OQ_W4, s.group, want_w1=s.center)
        act = oq.oq_quant_act(x, rot, s.afmt, center=s.center)
        w1 = wq["w1"] if s.center else None
        if s.afmt == oq.OQ_A4:
            y_sep = oq.oq_gemm_w4a4(oq.OQ_A4, act["codes"], act["scale"], wq["codes"], wq["scales"], N, s.group,
                                    mean=act["mean"], w1=w1)
        else:
            y_sep = oq.oq_gemm_w4a8(act["codes"], act["scale"], wq["codes"], wq["scales"], N, s.group,
                                    mean=act["mean"], w1=w1)
        y = oq.oq_linear_fused(x, rot, s.center, s.afmt, wq["codes"], wq["scales"], N, s.group, w1=w1)
    else:
        rot = oq.Rotation.dense32(to_dev(wl.t_act_bits))
        wq = oq.oq_quant_weight(to_dev(W), rot, oq.OQ_W_MXFP4, 32)
        act = oq.oq_quant_act(x, rot, oq.OQ_MXFP4)
        y_sep = oq.oq_gemm_w4a4(oq.OQ_MXFP4, act["codes"], act["e8m0"], wq["codes"], wq["scales"], N, 32)
        y = oq.oq_linear_fused(x, rot, False, oq.OQ_MXFP4, wq["codes"], wq["scales"], N, 32)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_sep.view(torch.int16)), "fused and separate calls differ"
    sel = slice(None) if rows is None else torch.as_tensor(rows, device="cuda")
    out = {"y": to_host(y[sel]), "wcodes": to_host(wq["codes"]), "wscales": to_host(wq["scales"]),
           "acodes": to_host(act["codes"][sel])}
    if s.rot == "rpbh":
        out["alpha"] = to_host(act["scale"][sel])
        out["mean"] = None if act["mean"] is None else to_host(act["mean"][sel])
        out["w1"] = None if not s.center else to_host(wq["w1"])
    else:
        out["e8m0"] = to_host(act["e8m0"][sel])
    return out


def _check_layer(wl, g, rows=None, wrows=None):
    s = wl.spec
    W = wl.weights[0]
    xb = wl.x_bits if rows is None else wl.x_bits[rows]
    if s.rot == "rpbh":
        wsel = slice(None) if wrows is None else wrows
        wref = OL.prepare_weight_rpbh(W[wsel], wl.perm, wl.signs, s.block, s.group)
        check_codes(OQ.unpack_int4(g["wcodes"][wsel]), wref["codes"], wref["flags"], "weight codes")
        np.testing.assert_array_equal(g["wscales"][wsel], wref["scales"])
        aref = OL.activations_int(xb, wl.perm, wl.signs, s.block, s.afmt, s.center)
        acodes = g["acodes"]
        acodes = OQ.unpack_int4(acodes.view(np.uint8)) if s.afmt == 4 else acodes.astype(np.int32)
        nm = check_codes(acodes, aref["codes"], aref["flags"], "activation codes")
        np.testing.assert_array_equal(g["alpha"], aref["alpha"])
        if s.center:
            np.testing.assert_array_equal(g["mean"], aref["mean"])
        # output rule on the GPU's own codes and scales
        act = {"codes": acodes, "alpha": g["alpha"], "mean": g["mean"]}
        wprep = {"codes": OQ.unpack_int4(g["wcodes"]), "scales": g["wscales"], "w1": g["w1"]}
        y_ref, S = OL.linear_int(act, wprep, s.group)
        frac = check_output(g["y"], y_ref, S, wl.K // s.group, "layer output")
    else:
        wsel = slice(None) if wrows is None else wrows
        wref = OL.prepare_weight_dense32(W[wsel], wl.t_act_bits)
        flags = wref["flags"] | np.repeat(wref["block_flags"], 32, axis=1)
        check_codes(OQ.unpack_nibbles(g["wcodes"][wsel]), wref["codes"], flags, "mx weight codes")
        aref = OL.activations_mx(xb, wl.t_act_bits)
        np.testing.assert_array_equal(g["e8m0"], aref["scale_bytes"])
        acodes = OQ.unpack_nibbles(g["acodes"])
        nm = check_codes(acodes, aref["codes"], aref["flags"], "mx activation codes")
        A = OQ.mx_dequant(acodes, g["e8m0"])
        Wd = OQ.mx_dequant(OQ.unpack_nibbles(g["wcodes"]), g["wscales"])
        y_ref, S = OG.gemm_mx(A, Wd)
        frac = check_output(g["y"], y_ref, S, wl.K // 32, "layer output")
    return nm, frac


@pytest.mark.parametrize("cid,M,N", [(1, 256, 1024), (2, 300, 256), (3, 260, 384), (4, 300, 256), (5, 200, 256)])
def test_layer_reduced(oq, cid, M, N):
    say("case layer reduced", cid, M, N)
    wl = WL.make_workload(cid, M=M, Ns=(N,))
    g = _gpu_layer(oq, wl)
    nm, frac = _check_layer(wl, g)
    say(f"  boundary code flips {nm}, outputs within 1 bf16 ulp {frac:.6f}")


@pytest.mark.parametrize("cid,n_index", [(1, 0), (2, 0), (2, 1), (3, 0), (3, 1), (4, 0), (5, 0)])
def test_layer_full_size_sampled(oq, cid, n_index):
    say("case layer full size", cid, n_index)
    spec = WL.config_spec(cid)
    wl = WL.make_workload(cid)
    if n_index:
        wl.weights[0] = wl.weights[n_index]
    rng = np.random.default_rng(cid)
    rows = np.unique(np.concatenate([[0, spec.M - 1], rng.choice(spec.M, 30, replace=False)]))
    wrows = np.unique(np.concatenate([[0], rng.choice(wl.weights[0].shape[0], 24, replace=False)]))
    g = _gpu_layer(oq, wl, 0, rows=rows)
    nm, frac = _check_layer_sampled(wl, g, rows, wrows)
    say(f"  sampled rows {len(rows)}: boundary code flips {nm}, within 1 bf16 ulp {frac:.6f}")


def _check_layer_sampled(wl, g, rows, wrows):
    sub = WL.LinearWorkload(wl.spec, len(rows), wl.K, wl.Ns, wl.x_bits[rows], wl.perm, wl.signs,
                            wl.t_act_bits, wl.weights)
    return _check_layer(sub, g, rows=None, wrows=wrows)
