"""Host side of the Lloyd-Max path (CPU only): the library's Newton solver for
the codebook against the oracle's root solve, the stored tables, and argument
validation of the Lloyd-Max entry points before anything is launched.

The fixed point of Lloyd's conditions is ill-conditioned at many levels (both
solvers reach residuals near 1e-11 at 40-digit precision, yet their float64
levels differ by up to ~1e-7 relative at 256 levels and d = 30720), so float64
levels are compared at 1e-6 and the float16 tables must be identical except
for a level the oracle places within 1e-6 (relative) of a float16 rounding
midpoint."""
import ctypes

import numpy as np
import pytest

from oracle import lloyd_max as LM


@pytest.fixture(scope="module")
def oq():
    import rotated_bit_quantized_amd as m
    return m


def _near_f16_midpoint(v):
    """True where float64 v lies within 1e-6 relative of a float16 midpoint."""
    h = v.astype(np.float16).astype(np.float64)
    up = np.nextafter(v.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(v.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    mids = np.stack([0.5 * (h + up), 0.5 * (h + dn)])
    return np.min(np.abs(mids - v), axis=0) <= 1e-6 * np.abs(v)


@pytest.mark.parametrize("d,bits", [(3, 4), (32, 4), (128, 8), (1024, 4), (1920, 6), (3072, 4), (3072, 8),
                                    (4096, 8), (30720, 4), (30720, 8), (257, 1), (48, 2)])
def test_codebook_matches_oracle(oq, d, bits):
    lv = oq.oq_lloyd_max_levels(d, bits)
    ref, res = LM.lloyd_max_levels(d, bits)
    assert res < 1e-11
    np.testing.assert_allclose(lv, ref, rtol=1e-6, atol=0)
    np.testing.assert_array_equal(lv, -lv[::-1])
    t16, thr = oq.oq_lloyd_max_tables(d, bits)
    r16, rthr = LM.codebook_tables(d, bits)
    same = t16 == r16.view(np.uint16)
    assert np.all(same | _near_f16_midpoint(ref))
    if np.all(same):
        np.testing.assert_array_equal(thr, rthr)


def test_solver_time_per_width(oq):
    """8-bit tables in well under the ~0.1 s per width the pages report."""
    import time
    t = time.perf_counter()
    oq.oq_lloyd_max_levels(30720, 8)
    assert time.perf_counter() - t < 0.5


def test_tables_rejects_bad_arguments(oq):
    with pytest.raises(oq.OQError):
        oq.oq_lloyd_max_levels(2, 4)
    with pytest.raises(oq.OQError):
        oq.oq_lloyd_max_levels(64, 9)
    with pytest.raises(oq.OQError):
        oq.oq_lloyd_max_levels(64, 0)


def test_lm_workspace_query(oq):
    assert oq.oq_workspace_bytes(oq.OQ_OP_GEMM_LM, 4096, 3072, 3072, 0) == 4096 * 3072 * 2
    assert oq.oq_workspace_bytes(oq.OQ_OP_GEMM_LM, 4096, 3072, 3072, oq.OQ_TILED) == 0
    assert oq.oq_workspace_bytes(oq.OQ_OP_GEMM_LM, 33, 64, 8, 0) == 64 * 64 * 2
    assert oq.oq_tiled_f16_bytes(33, 64) == 64 * 64 * 2
    assert oq.oq_tiled_f16_bytes(33, 40) == 0


def _err(oq):
    return oq.lib().oq_last_error().decode()


def test_lm_validation_rejects_before_launch(oq):
    lib = oq.lib()
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
    # bits out of range
    rc = lib.oq_quant_act_lm(fake, 4, 1024, 1024, None, 0, 9, 0, fake, fake, fake, 1024, fake, None, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED and "bits" in _err(oq)
    # width above the one-wavefront-per-row kernel
    rc = lib.oq_quant_act_lm(fake, 4, 8192, 8192, None, 0, 4, 0, fake, fake, fake, 4096, fake, None, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
    # missing codebook
    rc = lib.oq_quant_act_lm(fake, 4, 1024, 1024, None, 0, 4, 0, None, fake, fake, 512, fake, None, None)
    assert rc == oq.OQ_ERR_INVALID_ARG and "codebook" in _err(oq)
    # code rows too short for 8-bit indices
    rc = lib.oq_quant_act_lm(fake, 4, 1024, 1024, None, 0, 8, 0, fake, fake, fake, 512, fake, None, None)
    assert rc == oq.OQ_ERR_INVALID_ARG
    # centering without mean
    rc = lib.oq_quant_act_lm(fake, 4, 1024, 1024, None, 1, 4, 1, fake, fake, fake, 0, fake, None, None)
    assert rc == oq.OQ_ERR_INVALID_ARG
    # K not a multiple of 32
    rc = lib.oq_gemm_lm(4, 1, fake, 0, fake, 4, 48, None, fake, 64, None, None, None, fake, 64, None, 0, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
    # canonical codes without workspace
    rc = lib.oq_gemm_lm(4, 0, fake, 512, fake, 4, 1024, fake, fake, 64, None, None, None, fake, 64, None, 0, None)
    assert rc == oq.OQ_ERR_WORKSPACE
    # canonical codes without levels
    rc = lib.oq_gemm_lm(4, 0, fake, 512, fake, 4, 1024, None, fake, 64, None, None, None, fake, 64, fake, 1 << 24,
                        None)
    assert rc == oq.OQ_ERR_INVALID_ARG
    # mean without w1
    rc = lib.oq_gemm_lm(4, 1, fake, 0, fake, 4, 1024, None, fake, 64, fake, None, None, fake, 64, None, 0, None)
    assert rc == oq.OQ_ERR_INVALID_ARG
    # prepack group that does not divide K
    rc = lib.oq_prepack_w16(fake, fake, 64, 1024, 96, fake, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
