"""The C-ABI library loads and exports every entry point its header declares;
host-side validation rejects bad arguments before anything reaches a GPU.
No compute call is made here (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oq.h")


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def oq():
    import rotated_bit_quantized_amd as m
    return m


def test_header_symbols_exported(oq):
    names = _declared()
    assert "oq_linear_fused" in names and "oq_quant_act" in names
    lib = oq.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in oq.h but not exported by liboq.so"
    assert set(names) == set(oq.EXPORTED)


def test_workspace_query(oq):
    ws = oq.oq_workspace_bytes(oq.OQ_OP_LINEAR, 4096, 3072, 3072, oq.OQ_A4)
    # INT4 codes + scale + mean for 4096 tokens
    assert ws >= 4096 * 1536 + 2 * 4096 * 4 and ws % 256 == 0
    assert oq.oq_workspace_bytes(oq.OQ_OP_LINEAR, 0, 3072, 3072, oq.OQ_A4) >= 0
    assert oq.oq_workspace_bytes(99, 1, 64, 64, oq.OQ_A4) == 0


def _err(oq):
    return oq.lib().oq_last_error().decode()


def test_validation_rejects_before_launch(oq):
    lib = oq.lib()
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first
    # NULL activations
    rc = lib.oq_quant_act(None, 4, 1024, 1024, None, 0, oq.OQ_A8, fake, 1024, fake, None, None, None)
    assert rc == oq.OQ_ERR_INVALID_ARG and "x is NULL" in _err(oq)
    # width not a multiple of 16
    rc = lib.oq_quant_act(fake, 4, 1000, 1000, None, 0, oq.OQ_A8, fake, 1008, fake, None, None, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
    # misaligned rows
    rc = lib.oq_quant_act(fake, 4, 1024, 1028, None, 0, oq.OQ_A8, fake, 1024, fake, None, None, None)
    assert rc == oq.OQ_ERR_ALIGNMENT
    # bad block size
    rot = oq._binding.oq_rot(oq.OQ_ROT_RPBH, 1024, 96, 1, fake, fake, None)
    rc = lib.oq_quant_act(fake, 4, 1024, 1024, ctypes.byref(rot), 0, oq.OQ_A8, fake, 1024, fake, None, None, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED and "block" in _err(oq)
    # three rounds
    rot = oq._binding.oq_rot(oq.OQ_ROT_RPBH, 1024, 128, 3, fake, fake, None)
    rc = lib.oq_quant_act(fake, 4, 1024, 1024, ctypes.byref(rot), 0, oq.OQ_A8, fake, 1024, fake, None, None, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
    # MXFP4 without a dense transform
    rc = lib.oq_quant_act(fake, 4, 1024, 1024, None, 0, oq.OQ_MXFP4, fake, 512, None, fake, None, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
    # group that does not divide K
    rc = lib.oq_gemm_w4a8(fake, 1024, fake, 4, 1024, fake, fake, 64, 96, None, None, None, fake, 64, None, 0, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
    # mean without w1
    rc = lib.oq_gemm_w4a4(oq.OQ_A4, fake, 512, fake, 4, 1024, fake, fake, 64, 64, fake, None, None, fake, 64,
                          None, 0, None)
    assert rc == oq.OQ_ERR_INVALID_ARG
    # fused call without workspace
    rc = lib.oq_linear_fused(fake, 4, 1024, 1024, None, 0, oq.OQ_A8, fake, fake, 64, 128, None, None, fake, 64,
                             None, 0, None)
    assert rc == oq.OQ_ERR_WORKSPACE
    # unknown format
    rc = lib.oq_linear_fused(fake, 4, 1024, 1024, None, 0, 5, fake, fake, 64, 128, None, None, fake, 64,
                             fake, 1 << 20, None)
    assert rc == oq.OQ_ERR_INVALID_ARG


def test_binding_requires_device_tensors(oq):
    torch = pytest.importorskip("torch")
    x = torch.zeros((2, 64), dtype=torch.int16)
    with pytest.raises(oq.OQError):
        oq.oq_quant_act(x, None, oq.OQ_A8)


def test_tiled_gemm_rejects_operands_beyond_32bit_offsets(oq):
    # the tiled FP6 GEMM addresses each operand plane with 32-bit offsets; a
    # plane of 4 GiB or more is refused during validation (nothing launched)
    lib = oq._binding.lib()
    fake = ctypes.c_void_p(1 << 20)
    M, K, N = 1 << 22, 1536, 256          # oq_tiled_bytes(M, K) = 4.5 GiB
    assert oq.oq_tiled_bytes(M, K) >= 1 << 32
    rc = lib.oq_gemm_w4a4(oq.OQ_A4 | oq.OQ_TILED, fake, 0, fake, M, K, fake, fake, N, 64, None, None, None,
                          fake, N, None, 0, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED and "4 GiB" in _err(oq)
    rc = lib.oq_gemm_w4a4(oq.OQ_A4 | oq.OQ_TILED, fake, 0, fake, 256, K, fake, fake, M, 64, None, None, None,
                          fake, M, None, 0, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
    rc = lib.oq_gemm_w4a4_asym(oq.OQ_A4 | oq.OQ_TILED, fake, fake, fake, M, K, fake, fake, fake, N, None, None,
                               None, fake, N, None)
    assert rc == oq.OQ_ERR_UNSUPPORTED
