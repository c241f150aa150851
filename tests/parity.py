"""Comparison rules shared by the GPU parity tests.

Rules (the acceptance criteria of the layer, with the readings of the pages stated below):
  * integer codes and scale bytes: bit-exact, except elements the oracle flags
    as lying within 1e-6 relative of a rounding boundary; mismatches among
    flagged elements are counted and must stay below 1e-4 of all elements;
  * rotated float32 values: |g - v64| <= 1e-5 max(|v64|, rms_t) per element,
    and the count of elements differing from the canonical float32 value is
    reported (0 expected for the RPBH path);
  * bfloat16 outputs: |y - y*| <= ulp_bf16(y*) + (n + 3) 2^-24 S with y* the
    oracle's float64 epilogue rounded once, evaluated on the GPU's own codes.
"""
import numpy as np
import torch

from oracle import gemm as OG


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.cpu().numpy()


def check_codes(gpu, ref, flags, what):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    mism = gpu != ref
    bad = mism & ~np.asarray(flags, dtype=bool)
    assert not bad.any(), f"{what}: {int(bad.sum())} unflagged code mismatches, first at {np.argwhere(bad)[:5].tolist()}"
    frac = mism.sum() / max(1, mism.size)
    assert frac < 1e-4, f"{what}: flagged mismatch fraction {frac}"
    return int(mism.sum())


def check_rotated(g, v32, v64, what):
    g = np.asarray(g, dtype=np.float64)
    v64 = np.asarray(v64, dtype=np.float64)
    rms = np.sqrt(np.mean(v64 ** 2, axis=-1, keepdims=True))
    err = np.abs(g - v64) / np.maximum(np.abs(v64), np.maximum(rms, 1e-30))
    assert err.max() <= 1e-5, f"{what}: rotated value relative error {err.max()}"
    return int(np.sum(np.asarray(g, dtype=np.float32) != np.asarray(v32, dtype=np.float32)))


def check_output(y_gpu, y_ref, S, n_terms, what):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    tol = OG.output_tolerance(y_ref, S, n_terms)
    err = np.abs(y_gpu - y_ref.astype(np.float64))
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs outside tolerance; worst err {err.max()} "
                           f"at {np.unravel_index(np.argmax(err - tol), err.shape)}")
    within_ulp = np.mean(err <= OG.bf16_ulp(y_ref))
    return float(within_ulp)
