"""ctypes binding of liboq (include/oq.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
PyTorch tensors on a HIP device (PyTorch provides device memory and the
current stream); outputs that are not supplied are allocated with
``torch.empty``.  All arithmetic runs in the library's HIP kernels; there is
no other code path.  A non-zero status raises :class:`OQError`.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liboq.so")

OQ_OK, OQ_ERR_INVALID_ARG, OQ_ERR_UNSUPPORTED, OQ_ERR_ALIGNMENT, OQ_ERR_WORKSPACE, OQ_ERR_HIP = range(6)
OQ_ROT_RPBH, OQ_ROT_DENSE32, OQ_ROT_KRON = 1, 2, 3
OQ_A8, OQ_A6, OQ_A4, OQ_MXFP4 = 8, 6, 4, 0x104
OQ_W4, OQ_W_MXFP4 = 4, 0x104
OQ_OP_GEMM_W4A8, OQ_OP_GEMM_W4A4, OQ_OP_LINEAR, OQ_OP_GEMM_LM = 1, 2, 3, 4
OQ_TILED = 0x10000
OQ_SCALE_PCTL = 0x20000


class OQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[oq error {code}] {msg}")
        self.code = code


class oq_rot(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("rounds", ctypes.c_int32),
        ("perm", ctypes.c_void_p),
        ("signs", ctypes.c_void_p),
        ("mats", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"liboq.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "oq_last_error": ([], ctypes.c_char_p),
        "oq_center": ([vp, i64, i32, i64, vp, i64, vp, vp], ctypes.c_int),
        "oq_rotate": ([vp, vp, i64, i64, ctypes.c_int, vp, vp, i64, vp], ctypes.c_int),
        "oq_quant_act": ([vp, i64, i32, i64, vp, ctypes.c_int, ctypes.c_int, vp, i64, vp, vp, vp, vp], ctypes.c_int),
        "oq_quant_weight": ([vp, i32, i32, i64, vp, ctypes.c_int, i32, vp, vp, vp, vp], ctypes.c_int),
        "oq_gemm_w4a8": ([vp, i64, vp, i64, i32, vp, vp, i32, i32, vp, vp, vp, vp, i64, vp, sz, vp], ctypes.c_int),
        "oq_gemm_w4a4": ([ctypes.c_int, vp, i64, vp, i64, i32, vp, vp, i32, i32, vp, vp, vp, vp, i64, vp, sz, vp], ctypes.c_int),
        "oq_linear_fused": ([vp, i64, i32, i64, vp, ctypes.c_int, ctypes.c_int, vp, vp, i32, i32, vp, vp, vp, i64, vp, sz, vp], ctypes.c_int),
        "oq_probe_mfma": ([ctypes.c_int, i32, vp, ctypes.POINTER(ctypes.c_double), vp], ctypes.c_int),
        "oq_probe_sink_elems": ([], sz),
        "oq_linear_fused_noalloc": ([vp, i64, i32, i64, vp, ctypes.c_int, ctypes.c_int, vp, vp, i32, i32, vp, vp, vp,
                                     i64, vp], ctypes.c_int),
        "oq_workspace_bytes": ([ctypes.c_int, i64, i32, i32, ctypes.c_int], sz),
        "oq_tiled_bytes": ([i64, i32], sz),
        "oq_prepack_w4": ([vp, vp, i32, i32, i32, vp, vp, vp], ctypes.c_int),
        "oq_tiled_mx_bytes": ([i64, i32], sz),
        "oq_prepack_mx": ([vp, vp, i32, i32, vp, vp, vp], ctypes.c_int),
        "oq_lloyd_max_levels": ([i32, i32, vp], ctypes.c_int),
        "oq_lloyd_max_tables": ([i32, i32, vp, vp], ctypes.c_int),
        "oq_tiled_f16_bytes": ([i64, i32], sz),
        "oq_quant_act_lm": ([vp, i64, i32, i64, vp, ctypes.c_int, i32, ctypes.c_int, vp, vp, vp, i64, vp, vp, vp],
                            ctypes.c_int),
        "oq_prepack_w16": ([vp, vp, i32, i32, i32, vp, vp], ctypes.c_int),
        "oq_gemm_lm": ([i32, ctypes.c_int, vp, i64, vp, i64, i32, vp, vp, i32, vp, vp, vp, vp, i64, vp, sz, vp],
                       ctypes.c_int),
        "oq_quant_weight_asym": ([vp, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp], ctypes.c_int),
        "oq_prepack_w4_asym": ([vp, vp, vp, i32, i32, i32, vp, vp, vp, vp], ctypes.c_int),
        "oq_quant_act_gsum": ([vp, i64, i32, i64, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp], ctypes.c_int),
        "oq_gemm_w4a4_asym": ([ctypes.c_int, vp, vp, vp, i64, i32, vp, vp, vp, i32, vp, vp, vp, vp, i64, vp],
                              ctypes.c_int),
        "oq_kron_plan": ([i32, vp, vp, vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib = _load()
EXPORTED = ("oq_last_error", "oq_center", "oq_rotate", "oq_quant_act", "oq_quant_weight",
            "oq_gemm_w4a8", "oq_gemm_w4a4", "oq_linear_fused", "oq_workspace_bytes", "oq_tiled_bytes",
            "oq_prepack_w4", "oq_tiled_mx_bytes", "oq_prepack_mx", "oq_lloyd_max_levels", "oq_lloyd_max_tables",
            "oq_tiled_f16_bytes", "oq_quant_act_lm", "oq_prepack_w16", "oq_gemm_lm", "oq_quant_weight_asym",
            "oq_prepack_w4_asym", "oq_quant_act_gsum", "oq_gemm_w4a4_asym", "oq_kron_plan",
            "oq_linear_fused_noalloc", "oq_probe_mfma", "oq_probe_sink_elems")


def lib():
    return _lib


def _check(rc: int):
    if rc != OQ_OK:
        raise OQError(rc, _lib.oq_last_error().decode("utf-8", "replace"))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise OQError(OQ_ERR_INVALID_ARG, "tensors must live on the GPU")
    return t.device


def _need(t: Optional[torch.Tensor], nbytes: int, what: str, dtypes=None, optional: bool = False):
    """Argument check before a call: t is a GPU tensor of one of `dtypes`,
    contiguous, holding at least `nbytes` bytes (the library reads or writes
    that many from its base)."""
    if t is None:
        if optional:
            return
        raise OQError(OQ_ERR_INVALID_ARG, f"{what} is required")
    if not t.is_cuda:
        raise OQError(OQ_ERR_INVALID_ARG, f"{what} must live on the GPU")
    if dtypes is not None and t.dtype not in dtypes:
        raise OQError(OQ_ERR_INVALID_ARG, f"{what} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise OQError(OQ_ERR_INVALID_ARG, f"{what} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise OQError(OQ_ERR_INVALID_ARG, f"{what} holds {t.numel() * t.element_size()} bytes, {nbytes} needed")


_F32 = (torch.float32,)
_BYTES = (torch.uint8, torch.int8)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _out_y(y: Optional[torch.Tensor], M: int, N: int, dev) -> torch.Tensor:
    """The bfloat16 output [M][>= N] (allocated when not given)."""
    if y is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if (not y.is_cuda or y.dtype not in _BF16 or y.dim() != 2 or y.shape[0] < M or y.shape[1] < N
            or y.stride(1) != 1):
        raise OQError(OQ_ERR_INVALID_ARG, f"y must be a GPU bfloat16 matrix of at least {M} x {N} with unit column stride")
    return y


def _epilogue_args(M: int, N: int, mean, w1, bias):
    _need(mean, 4 * M, "mean", _F32, optional=True)
    _need(w1, 4 * N, "w1", _F32, optional=True)
    _need(bias, 4 * N, "bias", _F32, optional=True)


def _bits16(x: torch.Tensor) -> torch.Tensor:
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise OQError(OQ_ERR_INVALID_ARG, "bfloat16 input expected (or its 16-bit pattern)")
    return x


class Rotation:
    """Host descriptor plus the device arrays it points to (kept alive here)."""

    def __init__(self, kind: int, d: int, block: int = 0, rounds: int = 0, perm=None, signs=None, mats=None):
        self.kind, self.d, self.block, self.rounds = kind, d, block, rounds
        self.perm, self.signs, self.mats = perm, signs, mats
        self.c = oq_rot(kind, d, block, rounds, _p(perm), _p(signs), _p(mats))

    @staticmethod
    def rpbh(perm: torch.Tensor, signs: torch.Tensor, block: int) -> "Rotation":
        perm = perm.to(torch.int32).contiguous()
        signs = signs.to(torch.int8).contiguous()
        return Rotation(OQ_ROT_RPBH, perm.shape[-1], block, perm.shape[0], perm=perm, signs=signs)

    @staticmethod
    def kron(n: int) -> "Rotation":
        """The Paley x Sylvester rotation for native width n at the smallest
        admissible padded width (oq_kron_plan)."""
        m, b, npad = oq_kron_plan(n)
        return Rotation(OQ_ROT_KRON, n, b, m)

    @property
    def width(self) -> int:
        """Width of the rotated row (padded for the Kronecker rotation)."""
        return self.rounds * self.block if self.kind == OQ_ROT_KRON else self.d

    @staticmethod
    def dense32(mats_bits: torch.Tensor) -> "Rotation":
        """Per-32-block transforms T_b (bfloat16 bits [d/32][32][32]); the
        weight side uses their inverse-transposes, formed by the library."""
        d = mats_bits.shape[0] * 32
        return Rotation(OQ_ROT_DENSE32, d, 32, 1, mats=mats_bits.contiguous())

    def ref(self):
        return ctypes.byref(self.c)


def _rref(rot: Optional[Rotation]):
    return None if rot is None else rot.ref()


def oq_center(x, xc=None, mean=None):
    x = _bits16(x)
    M, d = x.shape
    dev = _dev(x)
    if mean is None:
        mean = torch.empty(M, dtype=torch.float32, device=dev)
    ldxc = 0 if xc is None else xc.stride(0)
    _check(_lib.oq_center(_p(x), M, d, x.stride(0), _p(xc), ldxc, _p(mean), _stream()))
    return xc, mean


def oq_rotate(rot: Rotation, x, center: bool = False, y=None, mean=None):
    x = _bits16(x)
    M = x.shape[0]
    dev = _dev(x)
    if y is None:
        y = torch.empty((M, rot.width), dtype=torch.float32, device=dev)
    if center and mean is None:
        mean = torch.empty(M, dtype=torch.float32, device=dev)
    _check(_lib.oq_rotate(rot.ref(), _p(x), M, x.stride(0), int(center), _p(mean), _p(y), y.stride(0), _stream()))
    return y, mean


def oq_quant_act(x, rot: Optional[Rotation], afmt: int, center: bool = False, codes=None, scale=None,
                 e8m0=None, mean=None):
    x = _bits16(x)
    M, d = x.shape
    dev = _dev(x)
    if rot is not None and rot.kind == OQ_ROT_KRON:
        d = rot.width  # codes have the padded width
    fmt = afmt & ~OQ_SCALE_PCTL  # the scale flag does not change the buffers
    mx_tiled = fmt == (OQ_MXFP4 | OQ_TILED)
    if codes is None and mx_tiled:
        codes = torch.empty(max(16, oq_tiled_mx_bytes(M, d)), dtype=torch.uint8, device=dev)
    elif codes is None and fmt & OQ_TILED:
        planes = 2 if (fmt & ~OQ_TILED) == OQ_A6 else 1
        codes = torch.empty(max(1, planes * oq_tiled_bytes(M, d)), dtype=torch.uint8, device=dev)
    elif codes is None:
        width = d if fmt in (OQ_A8, OQ_A6) else d // 2
        codes = torch.empty((M, width), dtype=torch.int8 if fmt in (OQ_A8, OQ_A6) else torch.uint8, device=dev)
    if mx_tiled:
        if e8m0 is None:
            e8m0 = torch.empty(max(4, oq_tiled_mx_bytes(M, d) // 16), dtype=torch.uint8, device=dev)
    elif fmt == OQ_MXFP4:
        if e8m0 is None:
            e8m0 = torch.empty((M, d // 32), dtype=torch.uint8, device=dev)
    elif scale is None:
        scale = torch.empty(M, dtype=torch.float32, device=dev)
    if center and mean is None:
        mean = torch.empty(M, dtype=torch.float32, device=dev)
    ldc = 0 if fmt & OQ_TILED else codes.stride(0) * codes.element_size()
    _check(_lib.oq_quant_act(_p(x), M, x.shape[1], x.stride(0), _rref(rot), int(center), afmt, _p(codes),
                             ldc, _p(scale), _p(e8m0), _p(mean), _stream()))
    return {"codes": codes, "scale": scale, "e8m0": e8m0, "mean": mean}


def oq_quant_weight(w, rot: Optional[Rotation], wfmt: int, group: int, codes=None, scales=None, w1=None,
                    want_w1: bool = False):
    N, K = w.shape
    dev = _dev(w)
    Kq = rot.width if rot is not None and rot.kind == OQ_ROT_KRON else K
    if codes is None:
        codes = torch.empty((N, Kq // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = (torch.empty((N, K // 32), dtype=torch.uint8, device=dev) if wfmt == OQ_W_MXFP4
                  else torch.empty((N, Kq // group), dtype=torch.float32, device=dev))
    if want_w1 and w1 is None:
        w1 = torch.empty(N, dtype=torch.float32, device=dev)
    _check(_lib.oq_quant_weight(_p(w), N, K, w.stride(0), _rref(rot), wfmt, group, _p(codes), _p(scales),
                                _p(w1), _stream()))
    return {"codes": codes, "scales": scales, "w1": w1}


def oq_gemm_w4a8(qa, a_scale, w, w_scale, N: int, group: int, mean=None, w1=None, bias=None, y=None,
                 ws=None):
    M, K = qa.shape
    if qa.dtype not in _BYTES or qa.stride(1) != 1:
        raise OQError(OQ_ERR_INVALID_ARG, "qa must be an int8 matrix with unit column stride")
    _need(a_scale, 4 * M, "a_scale", _F32)
    if M and N and group > 0:
        _need(w, N * K // 2, "w", _BYTES)
        _need(w_scale, 4 * N * (K // group), "w_scale", _F32)
    _epilogue_args(M, N, mean, w1, bias)
    _need(ws, 0, "ws", optional=True)
    y = _out_y(y, M, N, _dev(qa))
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.oq_gemm_w4a8(_p(qa), qa.stride(0), _p(a_scale), M, K, _p(w), _p(w_scale), N, group, _p(mean),
                             _p(w1), _p(bias), _p(y), y.stride(0), _p(ws), wsb, _stream()))
    return y


def oq_gemm_w4a4(afmt: int, qa, a_scale, w, w_scale, N: int, group: int, mean=None, w1=None, bias=None,
                 y=None, ws=None, M: Optional[int] = None, K: Optional[int] = None):
    if afmt & OQ_TILED:
        if M is None or K is None:
            raise OQError(OQ_ERR_INVALID_ARG, "tiled operands need explicit M and K")
        lda = 0
        if M > 0 and N > 0 and K > 0:
            if afmt == (OQ_MXFP4 | OQ_TILED):
                _need(qa, oq_tiled_mx_bytes(M, K), "qa", _BYTES)
                _need(a_scale, oq_tiled_mx_bytes(M, K) // 16, "a_scale", _BYTES)
                _need(w, oq_tiled_mx_bytes(N, K), "w", _BYTES)
                _need(w_scale, oq_tiled_mx_bytes(N, K) // 16, "w_scale", _BYTES)
            else:
                planes = 2 if (afmt & ~OQ_TILED) == OQ_A6 else 1
                _need(qa, planes * oq_tiled_bytes(M, K), "qa", _BYTES)
                _need(a_scale, 4 * M, "a_scale", _F32)
                _need(w, oq_tiled_bytes(N, K), "w", _BYTES)
                _need(w_scale, 4 * (K // 64) * ((N + 31) // 32 * 32), "w_scale", _F32)
    else:
        M = qa.shape[0]
        K = qa.shape[1] * 2
        lda = qa.stride(0) * qa.element_size()
        if qa.dtype not in _BYTES or qa.stride(1) != 1:
            raise OQError(OQ_ERR_INVALID_ARG, "qa must be a uint8 matrix with unit column stride")
        if M > 0 and N > 0:
            _need(w, N * K // 2, "w", _BYTES)
            if afmt == OQ_MXFP4:
                _need(a_scale, M * (K // 32), "a_scale", _BYTES)
                _need(w_scale, N * (K // 32), "w_scale", _BYTES)
            elif group > 0:
                _need(a_scale, 4 * M, "a_scale", _F32)
                _need(w_scale, 4 * N * (K // group), "w_scale", _F32)
    _epilogue_args(M, N, mean, w1, bias)
    y = _out_y(y, M, N, _dev(qa))
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.oq_gemm_w4a4(afmt, _p(qa), lda, _p(a_scale), M, K, _p(w),
                             _p(w_scale), N, group, _p(mean), _p(w1), _p(bias), _p(y), y.stride(0), _p(ws), wsb,
                             _stream()))
    return y


def oq_tiled_bytes(rows: int, K: int) -> int:
    return int(_lib.oq_tiled_bytes(rows, K))


def oq_prepack_w4(w, w_scale, N: int, K: int, group: int = 64, w_tiled=None, w_scale_t=None):
    dev = _dev(w)
    if w_tiled is None:
        w_tiled = torch.empty(max(1, oq_tiled_bytes(N, K)), dtype=torch.uint8, device=dev)
    if w_scale_t is None:
        w_scale_t = torch.empty((K // 64, (N + 31) // 32 * 32), dtype=torch.float32, device=dev)
    _check(_lib.oq_prepack_w4(_p(w), _p(w_scale), N, K, group, _p(w_tiled), _p(w_scale_t), _stream()))
    return {"codes": w_tiled, "scales": w_scale_t}


def oq_tiled_mx_bytes(rows: int, K: int) -> int:
    return int(_lib.oq_tiled_mx_bytes(rows, K))


def oq_prepack_mx(w, w_e8m0, N: int, K: int, w_tiled=None, w_e8m0_tiled=None):
    dev = _dev(w)
    nb = oq_tiled_mx_bytes(N, K)
    if w_tiled is None:
        w_tiled = torch.empty(max(16, nb), dtype=torch.uint8, device=dev)
    if w_e8m0_tiled is None:
        w_e8m0_tiled = torch.empty(max(4, nb // 16), dtype=torch.uint8, device=dev)
    _check(_lib.oq_prepack_mx(_p(w), _p(w_e8m0), N, K, _p(w_tiled), _p(w_e8m0_tiled), _stream()))
    return {"codes": w_tiled, "scales": w_e8m0_tiled}


def oq_workspace_bytes(op: int, M: int, K: int, N: int, afmt: int) -> int:
    return int(_lib.oq_workspace_bytes(op, M, K, N, afmt))


def oq_linear_fused(x, rot: Optional[Rotation], center: bool, afmt: int, w, w_scale, N: int, group: int,
                    w1=None, bias=None, y=None, ws=None):
    x = _bits16(x)
    M, K = x.shape
    dev = _dev(x)
    fmt = afmt & ~OQ_SCALE_PCTL
    if M > 0 and N > 0:
        if fmt == (OQ_MXFP4 | OQ_TILED):
            _need(w, oq_tiled_mx_bytes(N, K), "w", _BYTES)
            _need(w_scale, oq_tiled_mx_bytes(N, K) // 16, "w_scale", _BYTES)
        elif fmt & OQ_TILED:
            _need(w, oq_tiled_bytes(N, K), "w", _BYTES)
            _need(w_scale, 4 * (K // 64) * ((N + 31) // 32 * 32), "w_scale", _F32)
        else:
            _need(w, N * K // 2, "w", _BYTES)
            if fmt == OQ_MXFP4:
                _need(w_scale, N * (K // 32), "w_scale", _BYTES)
            elif group > 0:
                _need(w_scale, 4 * N * (K // group), "w_scale", _F32)
    _epilogue_args(M, N, None, w1, bias)
    y = _out_y(y, M, N, dev)
    if ws is None:
        ws = torch.empty(max(1, oq_workspace_bytes(OQ_OP_LINEAR, M, K, N, afmt)), dtype=torch.uint8, device=dev)
    _check(_lib.oq_linear_fused(_p(x), M, K, x.stride(0), _rref(rot), int(center), afmt, _p(w), _p(w_scale), N,
                                group, _p(w1), _p(bias), _p(y), y.stride(0), _p(ws), ws.numel(), _stream()))
    return y


OQ_PROBE_FP6, OQ_PROBE_FP4, OQ_PROBE_FP8, OQ_PROBE_I8, OQ_PROBE_BF16, OQ_PROBE_F16 = 1, 2, 3, 4, 5, 6
OQ_PROBE_FP6_UPDATE = 7


def oq_probe_mfma(kind: int, iters: int, sink=None):
    """Launches the matrix-core rate probe on the current stream; returns
    (operation count of the launch, sink).  The caller times it."""
    if sink is None:
        sink = torch.empty(int(_lib.oq_probe_sink_elems()), dtype=torch.float32, device="cuda")
    _need(sink, 4 * int(_lib.oq_probe_sink_elems()), "sink", _F32)
    ops = ctypes.c_double(0.0)
    _check(_lib.oq_probe_mfma(kind, iters, _p(sink), ctypes.byref(ops), _stream()))
    return ops.value, sink


OQ_NOALLOC_SCRATCH_BYTES = 32 << 20


def oq_linear_fused_noalloc(x, rot: Optional[Rotation], center: bool, afmt: int, w, w_scale, N: int, group: int,
                            w1=None, bias=None, y=None):
    """oq_linear_fused without a workspace: the library's static per-GPU
    scratch holds the codes (calls on one GPU must not overlap)."""
    x = _bits16(x)
    M, K = x.shape
    dev = _dev(x)
    _epilogue_args(M, N, None, w1, bias)
    y = _out_y(y, M, N, dev)
    _check(_lib.oq_linear_fused_noalloc(_p(x), M, K, x.stride(0), _rref(rot), int(center), afmt, _p(w), _p(w_scale),
                                        N, group, _p(w1), _p(bias), _p(y), y.stride(0), _stream()))
    return y


# ---------------------------------------------------------------- Lloyd-Max path
def oq_lloyd_max_levels(d: int, bits: int) -> np.ndarray:
    """Host call: float64 levels [2^bits] of the Lloyd-Max codebook for width d."""
    out = np.zeros(1 << bits, dtype=np.float64)
    _check(_lib.oq_lloyd_max_levels(d, bits, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def oq_lloyd_max_tables(d: int, bits: int):
    """Host call: (float16 level bits uint16 [2^bits], float32 thresholds [2^bits - 1])."""
    lv = np.zeros(1 << bits, dtype=np.uint16)
    thr = np.zeros((1 << bits) - 1, dtype=np.float32)
    _check(_lib.oq_lloyd_max_tables(d, bits, lv.ctypes.data_as(ctypes.c_void_p),
                                    thr.ctypes.data_as(ctypes.c_void_p)))
    return lv, thr


def oq_tiled_f16_bytes(rows: int, K: int) -> int:
    return int(_lib.oq_tiled_f16_bytes(rows, K))


def oq_quant_act_lm(x, rot: Optional[Rotation], bits: int, levels, thresholds, tiled: bool = False,
                    center: bool = False, codes=None, scale=None, mean=None):
    """levels: device uint16/int16 float16 bits [2^bits]; thresholds: device float32."""
    x = _bits16(x)
    M, d = x.shape
    dev = _dev(x)
    if codes is None and tiled:
        codes = torch.empty(max(16, oq_tiled_f16_bytes(M, d)), dtype=torch.uint8, device=dev)
    elif codes is None:
        codes = torch.empty((M, d // 2 if bits <= 4 else d), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(M, dtype=torch.float32, device=dev)
    if center and mean is None:
        mean = torch.empty(M, dtype=torch.float32, device=dev)
    ldc = 0 if tiled else codes.stride(0) * codes.element_size()
    _check(_lib.oq_quant_act_lm(_p(x), M, d, x.stride(0), _rref(rot), int(center), bits, int(tiled), _p(levels),
                                _p(thresholds), _p(codes), ldc, _p(scale), _p(mean), _stream()))
    return {"codes": codes, "scale": scale, "mean": mean}


def oq_prepack_w16(w, w_scale, N: int, K: int, group: int, w16=None):
    dev = _dev(w)
    if w16 is None:
        w16 = torch.empty(max(16, oq_tiled_f16_bytes(N, K)) // 2, dtype=torch.int16, device=dev)
    _check(_lib.oq_prepack_w16(_p(w), _p(w_scale), N, K, group, _p(w16), _stream()))
    return w16


def oq_gemm_lm(bits: int, qa, a_scale, w16, N: int, levels=None, tiled: bool = False, mean=None, w1=None,
               bias=None, y=None, ws=None, M: Optional[int] = None, K: Optional[int] = None):
    if tiled:
        if M is None or K is None:
            raise OQError(OQ_ERR_INVALID_ARG, "tiled operands need explicit M and K")
        lda = 0
        if M > 0 and N > 0 and K > 0:
            _need(qa, oq_tiled_f16_bytes(M, K), "qa")
    else:
        M = qa.shape[0]
        K = qa.shape[1] * (2 if bits <= 4 else 1)
        lda = qa.stride(0) * qa.element_size()
        if ws is None:
            ws = torch.empty(max(16, oq_workspace_bytes(OQ_OP_GEMM_LM, M, K, N, 0)), dtype=torch.uint8,
                             device=_dev(qa))
    if M > 0 and N > 0 and K > 0:
        _need(a_scale, 4 * M, "a_scale", _F32)
        _need(w16, oq_tiled_f16_bytes(N, K), "w16")
    _epilogue_args(M, N, mean, w1, bias)
    y = _out_y(y, M, N, _dev(qa))
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.oq_gemm_lm(bits, int(tiled), _p(qa), lda, _p(a_scale), M, K, _p(levels), _p(w16), N, _p(mean),
                           _p(w1), _p(bias), _p(y), y.stride(0), _p(ws), wsb, _stream()))
    return y


# ---------------------------------------------------------------- asymmetric weights
def oq_quant_weight_asym(w, rot: Optional[Rotation], group: int, codes=None, sigma=None, zero=None, w1=None,
                         want_w1: bool = False):
    N, K = w.shape
    dev = _dev(w)
    Kq = rot.width if rot is not None and rot.kind == OQ_ROT_KRON else K
    if codes is None:
        codes = torch.empty((N, Kq // 2), dtype=torch.uint8, device=dev)
    if sigma is None:
        sigma = torch.empty((N, Kq // group), dtype=torch.int16, device=dev)
    if zero is None:
        zero = torch.empty((N, Kq // group), dtype=torch.int16, device=dev)
    if want_w1 and w1 is None:
        w1 = torch.empty(N, dtype=torch.float32, device=dev)
    _check(_lib.oq_quant_weight_asym(_p(w), N, K, w.stride(0), _rref(rot), group, _p(codes), _p(sigma), _p(zero),
                                     _p(w1), _stream()))
    return {"codes": codes, "sigma": sigma, "zero": zero, "w1": w1}


def oq_prepack_w4_asym(w, sigma, zero, N: int, K: int, group: int = 64):
    dev = _dev(w)
    Np = (N + 31) // 32 * 32
    w_tiled = torch.empty(max(16, oq_tiled_bytes(N, K)), dtype=torch.uint8, device=dev)
    w_scale_t = torch.empty((K // 64, Np), dtype=torch.float32, device=dev)
    corr = torch.empty((K // 64, Np, 2), dtype=torch.int32, device=dev)
    _check(_lib.oq_prepack_w4_asym(_p(w), _p(sigma), _p(zero), N, K, group, _p(w_tiled), _p(w_scale_t), _p(corr),
                                   _stream()))
    return {"codes": w_tiled, "scales": w_scale_t, "corr": corr}


def oq_quant_act_gsum(x, rot: Optional[Rotation], afmt: int, center: bool = False, codes=None, scale=None,
                      gsum=None, mean=None):
    x = _bits16(x)
    M, d = x.shape
    dev = _dev(x)
    fmt = afmt & ~OQ_SCALE_PCTL
    if codes is None:
        planes = 2 if (fmt & ~OQ_TILED) == OQ_A6 else 1
        codes = torch.empty(max(16, planes * oq_tiled_bytes(M, d)), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(M, dtype=torch.float32, device=dev)
    if gsum is None:  # one word per (group, row): two bfloat16 pieces of the group sum
        gsum = torch.empty((d // 64, M), dtype=torch.int32, device=dev)
    if center and mean is None:
        mean = torch.empty(M, dtype=torch.float32, device=dev)
    _check(_lib.oq_quant_act_gsum(_p(x), M, d, x.stride(0), _rref(rot), int(center), afmt, _p(codes), _p(scale),
                                  _p(gsum), _p(mean), _stream()))
    return {"codes": codes, "scale": scale, "gsum": gsum, "mean": mean}


def oq_gemm_w4a4_asym(qa, a_scale, gsum, w, N: int, M: int, K: int, mean=None, w1=None, bias=None, y=None,
                      afmt: int = OQ_A4 | OQ_TILED):
    """w: oq_prepack_w4_asym output (dict with codes, scales, corr)."""
    if M > 0 and N > 0 and K > 0:
        Np = (N + 31) // 32 * 32
        _need(qa, oq_tiled_bytes(M, K), "qa", _BYTES)
        _need(a_scale, 4 * M, "a_scale", _F32)
        _need(gsum, 4 * (K // 64) * M, "gsum")
        _need(w["codes"], oq_tiled_bytes(N, K), "w codes", _BYTES)
        _need(w["scales"], 4 * (K // 64) * Np, "w scales", _F32)
        _need(w["corr"], 8 * (K // 64) * Np, "w corr")
    _epilogue_args(M, N, mean, w1, bias)
    y = _out_y(y, M, N, _dev(qa))
    _check(_lib.oq_gemm_w4a4_asym(afmt, _p(qa), _p(a_scale), _p(gsum), M, K, _p(w["codes"]), _p(w["scales"]),
                                  _p(w["corr"]), N, _p(mean), _p(w1), _p(bias), _p(y), y.stride(0), _stream()))
    return y


def oq_kron_plan(n: int):
    """Host call: (m, block, n_pad), the smallest admissible padded width."""
    m, b, p = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.oq_kron_plan(n, ctypes.byref(m), ctypes.byref(b), ctypes.byref(p)))
    return m.value, b.value, p.value
