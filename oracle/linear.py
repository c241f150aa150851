"""Offline weight preparation and the whole rotated low-bit linear forward pass.

Parity pins: tests/test_oracle_gemm.py (the forward pass, w_1, the offset
invariance) and tests/test_oracle_rotation.py (the weight-side transform).

Sources:
  CentriQ Sec. 3 "Hadamard rotation" (W x = (W H^T)(H x): the rotation is
  folded into the weight offline), Sec. 4.2 Eq. 4 (w_1 = W 1 computed once in
  FP32 from the unquantized weight), Eq. 5 (forward pass), App. B.1 (the
  weight absorbs the rotation offline as W P^T H^T).
  WUSH review, "Core claim": weights take the inverse-transpose of the
  activation transform.
  OrbitQuant PR #25 "Default changes": absmax INT8 at A8; the configurations
  also use 6- and 4-bit absmax codes (Eq. 1 with b = 6, 4).
  CentriQ Sec. 4.2 "Scale and grid": the percentile range in place of absmax.
"""
from __future__ import annotations

import math

import numpy as np

from . import gemm, quant, rotation


def row_sums_fp32(W: np.ndarray) -> np.ndarray:
    """w_1 = RN32(W 1), the exact row sum rounded once."""
    W = np.asarray(W, dtype=np.float64)
    return np.array([math.fsum(r) for r in W], dtype=np.float64).astype(np.float32)


def prepare_weight_rpbh(W, perm, signs, block, group):
    """Fold R into W (row o -> R w_o, canonical float32 order), quantize to
    symmetric INT4 per group, pack; w_1 from the unrotated, unquantized W."""
    wr = rotation.rpbh_fp32(np.asarray(W, dtype=np.float32), perm, signs, block)
    q, s, flag = quant.quant_groups_int(wr, group, 7)
    return {"rotated": wr, "codes": q, "scales": s, "flags": flag,
            "packed": quant.pack_int4(q), "w1": row_sums_fp32(W)}


def prepare_weight_dense32(W, t_act_bits):
    """w'_b = T_w,b w_b per 32-block with T_w,b = T_b^{-T} formed here from the
    stored bfloat16 activation transforms (WUSH review, "Core claim"), in
    float64 and rounded once to float32, then MXFP4."""
    t_w = rotation.dense32_weight_transform(t_act_bits)
    wr = rotation.dense32_fp64(np.asarray(W, dtype=np.float32), t_w).astype(np.float32)
    codes, sb, eflag, bflag = quant.quant_mx(wr)
    return {"rotated": wr, "codes": codes, "scale_bytes": sb, "flags": eflag,
            "block_flags": bflag, "packed": quant.pack_nibbles(codes)}


def activations_int(x_bits, perm, signs, block, afmt_bits, center, pctl=False):
    """Online activation path: (mean) -> (center) -> RPBH -> absmax codes, or
    percentile-scaled codes (CentriQ Sec. 4.2 "Scale and grid") with pctl."""
    x32 = quant.bf16_to_f32(x_bits)
    m = None
    if center:
        m = quant.token_mean(x32)
        x32 = quant.center(x32, m)
    v = rotation.rpbh_fp32(x32, perm, signs, block) if perm is not None else x32
    quantize = quant.quant_token_pctl if pctl else quant.quant_token_int
    q, alpha, flag = quantize(v, quant.qmax_for_bits(afmt_bits))
    return {"mean": m, "rotated": v, "codes": q, "alpha": alpha, "flags": flag}


def activations_mx(x_bits, t_act_bits):
    x32 = quant.bf16_to_f32(x_bits)
    T = quant.bf16_to_f32(t_act_bits)
    v, n_int = rotation.dense32_fp32(x32, T)
    codes, sb, eflag, bflag = quant.quant_mx(v)
    return {"rotated": v, "codes": codes, "scale_bytes": sb, "flags": eflag,
            "block_flags": bflag, "packed": quant.pack_nibbles(codes), "exact_int_sums": n_int}


def linear_int(act, wprep, group, bias=None):
    """y* and S for the integer path given activation and weight results."""
    acc = gemm.group_acc(act["codes"], wprep["codes"], group)
    mean = act["mean"]
    return gemm.epilogue_int(act["alpha"], acc, wprep["scales"],
                             mean, wprep["w1"] if mean is not None else None, bias)


def linear_mx(act, wprep, bias=None):
    A = quant.mx_dequant(act["codes"], act["scale_bytes"])
    W = quant.mx_dequant(wprep["codes"], wprep["scale_bytes"])
    return gemm.gemm_mx(A, W, bias)
