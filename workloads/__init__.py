"""Seeded synthetic inputs for the rotated low-bit linear layer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation is applied, nothing is quantized, packed or
multiplied here).  Both the CPU oracle and the HIP path consume exactly the
arrays produced here.

Workloads follow the shapes and value distributions of the five rotated-linear
settings studied on the pages (OrbitQuant PR #25 "Default changes" and
"Benchmark subsets"; CentriQ Sec. 4.2 and Eq. 4; WUSH review "Core claim"):

  c1  W4A8 single linear        256 x 1024 -> 1024,  RPBH h=128, 1 round
  c2  W4A4 DiT width            4096 x 3072 -> 3072 and -> 12288, h=1024
  c3  W4A6 non-power-of-two     4096 x 1920 -> 1920 and -> 7680, h=128, 2 rounds
  c4  centered W4A4 (adaLN)     4096 x 3072 -> 3072, exact mean + rank-1 restore
  c5  MXFP4 W4A4 LLM shape      8192 x 4096 -> 14336, dense per-32 transforms

Seeds: ``numpy.random.Generator(PCG64(SeedSequence([config_id, stream])))``
with fixed stream numbers (0 activations, 1 and 11 weights of the first and
second linear, 2 outlier channels, 3/4 permutation/signs of the first
rotation round, 5/6 of the second, 7/8 the dense transform's diagonal and
orthogonal factor, 9 the per-token adaLN mean and gain).

Bit conventions (inputs are defined by their bits):
  * activations: drawn in float64, rounded to float32 (nearest), then to
    bfloat16 (nearest-even); returned as uint16 bit patterns;
  * weights: float32;
  * permutation: int32 [rounds][d], used as a gather u[i] = v[perm[i]];
  * signs: int8 [rounds][d] in {-1, +1};
  * dense transforms: bfloat16 bits [d/32][32][32] row-major (the activation
    side; the weight side is derived from them by whoever consumes them).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "LinearWorkload",
    "CONFIGS",
    "config_spec",
    "make_workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "rng_for",
]

# activation formats (numerically identical to the C header's enum values)
A8, A6, A4, MXFP4 = 8, 6, 4, 0x104

STREAM_X, STREAM_W0, STREAM_OUTLIER = 0, 1, 2
STREAM_PERM1, STREAM_SIGN1, STREAM_PERM2, STREAM_SIGN2 = 3, 4, 5, 6
STREAM_T_DIAG, STREAM_T_ORTH, STREAM_ADALN = 7, 8, 9
STREAM_W1 = 11


def rng_for(config_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, stream])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    cid: int
    name: str
    M: int
    K: int
    Ns: tuple
    act: str            # "outliers20", "student_t", "gauss", "adaln", "outliers30"
    rot: str            # "rpbh" | "dense32"
    block: int
    rounds: int
    afmt: int
    group: int
    center: bool


CONFIGS = {
    1: ConfigSpec(1, "c1_w4a8_256x1024", 256, 1024, (1024,), "outliers20", "rpbh", 128, 1, A8, 128, False),
    2: ConfigSpec(2, "c2_w4a4_dit_4096x3072", 4096, 3072, (3072, 12288), "student_t", "rpbh", 1024, 1, A4, 64, False),
    3: ConfigSpec(3, "c3_w4a6_4096x1920_2rounds", 4096, 1920, (1920, 7680), "gauss", "rpbh", 128, 2, A6, 64, False),
    4: ConfigSpec(4, "c4_centered_w4a4_4096x3072", 4096, 3072, (3072,), "adaln", "rpbh", 1024, 1, A4, 64, True),
    5: ConfigSpec(5, "c5_mxfp4_8192x4096x14336", 8192, 4096, (14336,), "outliers30", "dense32", 32, 1, MXFP4, 32, False),
}


def config_spec(cid: int) -> ConfigSpec:
    return CONFIGS[cid]


@dataclasses.dataclass
class LinearWorkload:
    spec: ConfigSpec
    M: int
    K: int
    Ns: tuple
    x_bits: np.ndarray                 # uint16 [M, K] bfloat16 bits
    perm: Optional[np.ndarray]         # int32 [rounds, K]
    signs: Optional[np.ndarray]        # int8 [rounds, K]
    t_act_bits: Optional[np.ndarray]   # uint16 [K/32, 32, 32] bfloat16 bits
    weights: list                      # float32 [N, K] per linear

    @property
    def x_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.x_bits)


def _activations(spec: ConfigSpec, M: int, K: int) -> np.ndarray:
    g = rng_for(spec.cid, STREAM_X)
    z = g.standard_normal((M, K))
    if spec.act == "outliers20":
        ch = rng_for(spec.cid, STREAM_OUTLIER).choice(K, 4, replace=False)
        z[:, ch] *= 20.0
    elif spec.act == "outliers30":
        n = int(round(0.005 * K))
        ch = rng_for(spec.cid, STREAM_OUTLIER).choice(K, n, replace=False)
        z[:, ch] *= 30.0
    elif spec.act == "student_t":
        # heavy tails on 1% of channels: those channels are *replaced* by t(3) draws
        n = int(round(0.01 * K))
        go = rng_for(spec.cid, STREAM_OUTLIER)
        ch = go.choice(K, n, replace=False)
        z[:, ch] = go.standard_t(3.0, size=(M, n))
    elif spec.act == "adaln":
        ga = rng_for(spec.cid, STREAM_ADALN)
        mu = ga.normal(0.0, 3.0, size=(M, 1))
        gamma = ga.uniform(-0.5, 0.5, size=(M, 1))
        z = (1.0 + gamma) * z + mu
    elif spec.act == "gauss":
        pass
    else:
        raise ValueError(spec.act)
    return f32_to_bf16_bits(z.astype(np.float32))


def _rotation_metadata(spec: ConfigSpec, K: int):
    perms, signs = [], []
    for r in range(spec.rounds):
        sp, ss = (STREAM_PERM1, STREAM_SIGN1) if r == 0 else (STREAM_PERM2, STREAM_SIGN2)
        perms.append(rng_for(spec.cid, sp).permutation(K).astype(np.int32))
        signs.append(np.where(rng_for(spec.cid, ss).integers(0, 2, size=K) == 1, 1, -1).astype(np.int8))
    return np.stack(perms), np.stack(signs)


def _dense32_mats(spec: ConfigSpec, K: int):
    """Seeded per-32-block transforms T_b = (H32/sqrt 32) diag(s_b) Q_b with
    s_b log-uniform on [0.5, 2] and Q_b Haar orthogonal, stored as bfloat16."""
    from scipy.linalg import hadamard  # library construction of the +-1 Sylvester matrix
    nb = K // 32
    gd = rng_for(spec.cid, STREAM_T_DIAG)
    go = rng_for(spec.cid, STREAM_T_ORTH)
    h = hadamard(32).astype(np.float64) / np.sqrt(32.0)
    t_bits = np.empty((nb, 32, 32), dtype=np.uint16)
    for b in range(nb):
        s = np.exp(gd.uniform(np.log(0.5), np.log(2.0), size=32))
        a = go.standard_normal((32, 32))
        q, r = np.linalg.qr(a)
        q = q * np.sign(np.diag(r))[None, :]
        t_bits[b] = f32_to_bf16_bits((h @ np.diag(s) @ q).astype(np.float32))
    return t_bits


def make_workload(cid: int, M: Optional[int] = None, K: Optional[int] = None,
                  Ns: Optional[tuple] = None, n_linears: Optional[int] = None) -> LinearWorkload:
    """Build config ``cid``; M/K/Ns may be overridden for reduced test sizes
    (K must stay a multiple of the block and of the weight group)."""
    spec = CONFIGS[cid]
    M = spec.M if M is None else int(M)
    K = spec.K if K is None else int(K)
    Ns = tuple(spec.Ns if Ns is None else Ns)
    if n_linears is not None:
        Ns = Ns[:n_linears]
    if K % spec.block or K % spec.group:
        raise ValueError("K must be a multiple of the block and the group")
    x_bits = _activations(spec, M, K)
    perm = signs = t_bits = None
    if spec.rot == "rpbh":
        perm, signs = _rotation_metadata(spec, K)
    else:
        t_bits = _dense32_mats(spec, K)
    weights = []
    for i, n in enumerate(Ns):
        gw = rng_for(spec.cid, STREAM_W0 if i == 0 else STREAM_W1 + (i - 1) * 10)
        weights.append(gw.normal(0.0, 0.02, size=(n, K)).astype(np.float32))
    return LinearWorkload(spec, M, K, Ns, x_bits, perm, signs, t_bits, weights)
