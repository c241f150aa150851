"""Pins of oracle/quant.py (CPU only)."""
import numpy as np
import pytest

from conftest import read_golden
from oracle import quant as Q


def test_absmax_codes_golden():
    for ln in read_golden("absmax_codes.txt"):
        bits, vals, codes, alpha = [p.strip() for p in ln.split("|")]
        v = np.array([float(t) for t in vals.split()], dtype=np.float32)
        q, a, _ = Q.quant_token_int(v[None, :], Q.qmax_for_bits(int(bits)))
        np.testing.assert_array_equal(q[0], [int(t) for t in codes.split()])
        assert float(a[0]) == float(alpha)


@pytest.mark.parametrize("qmax", [127, 31, 7])
def test_quantizer_properties(qmax):
    rng = np.random.default_rng(20)
    v = (rng.standard_normal((64, 512)) * rng.uniform(0.01, 50, size=(64, 1))).astype(np.float32)
    q, alpha, _ = Q.quant_token_int(v, qmax)
    assert q.min() >= -qmax and q.max() <= qmax
    # the absmax element maps to exactly +-qmax
    j = np.argmax(np.abs(v), axis=1)
    np.testing.assert_array_equal(np.abs(q[np.arange(64), j]), qmax)
    # reconstruction error at most half a step (plus float32 rounding)
    err = np.abs(v.astype(np.float64) - alpha[:, None].astype(np.float64) * q)
    assert np.all(err <= alpha[:, None] * (0.5 + 1e-5))
    # alpha qmax reproduces the range to float32 rounding
    np.testing.assert_allclose(alpha * qmax, np.abs(v).max(axis=1), rtol=2e-7)
    # scaling a token by a power of two leaves its codes unchanged
    q2, alpha2, _ = Q.quant_token_int((v * np.float32(8.0)).astype(np.float32), qmax)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(alpha2, alpha * np.float32(8.0))


def test_zero_token_uses_epsilon():
    # model card "Quantization": activation normalization epsilon 1e-10
    q, alpha, _ = Q.quant_token_int(np.zeros((2, 64), dtype=np.float32), 7)
    assert np.all(q == 0)
    assert alpha[0] == np.float32(np.float32(1e-10) / np.float32(7))


def test_boundary_flags():
    v = np.array([[7.0, 1.5, 2.5000003, 0.3]], dtype=np.float32)
    q, _, flag = Q.quant_token_int(v, 7)
    # scaled values are the inputs themselves (a = 7): 1.5 and 2.5000003
    # sit on or within 1e-6 of a half-integer; 7 and 0.3 do not
    np.testing.assert_array_equal(flag[0], [False, True, True, False])
    np.testing.assert_array_equal(q[0], [7, 2, 3, 0])


def test_int4_pack_golden_and_exhaustive():
    for ln in read_golden("int4_pack.txt"):
        a, b, byte = ln.split()
        assert Q.pack_int4(np.array([int(a), int(b)]))[0] == int(byte, 16)
    allb = np.arange(256, dtype=np.uint8)
    u = Q.unpack_int4(allb[None, :])[0]
    assert u.min() == -8 and u.max() == 7
    np.testing.assert_array_equal(Q.pack_int4(u[None, :])[0], allb)


def test_group_quantizer_matches_token_quantizer_per_group():
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    q, s, _ = Q.quant_groups_int(w, 64, 7)
    for g in range(4):
        qq, aa, _ = Q.quant_token_int(w[:, g * 64:(g + 1) * 64], 7)
        np.testing.assert_array_equal(q[:, g * 64:(g + 1) * 64], qq)
        np.testing.assert_array_equal(s[:, g], aa)


def test_mean_is_exact_sum_rounded_once():
    x = np.array([[1.0, 2.0, 3.0, 4.0], [2.0 ** 20, 1.0, -(2.0 ** 20), 2.0 ** -10]], dtype=np.float32)
    m = Q.token_mean(x)
    assert m[0] == np.float32(2.5)
    assert m[1] == np.float32((1.0 + 2.0 ** -10) / 4.0)
    xc = Q.center(x, m)
    assert xc.dtype == np.float32
    np.testing.assert_array_equal(xc[0], [-1.5, -0.5, 0.5, 1.5])
    assert Q.fp64_sum_is_exact(x)
    assert not Q.fp64_sum_is_exact(np.array([[2.0 ** 60, 2.0 ** -60]], dtype=np.float32))


def test_centered_sum_near_zero():
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((16, 3072)) * 2 + rng.normal(0, 3, size=(16, 1))).astype(np.float32)
    xc = Q.center(x, Q.token_mean(x))
    # each centered coordinate carries at most half an ulp of rounding
    bound = 3072 * np.max(np.abs(x)) * 2.0 ** -24
    assert np.all(np.abs(xc.astype(np.float64).sum(axis=1)) <= bound)


def test_e2m1_table_golden():
    for ln in read_golden("e2m1_values.txt"):
        code, val = ln.split()
        c = int(code, 16)
        dec = Q.e2m1_decode(np.array([c]))[0]
        assert dec == float(val)
        # encode(decode(c)) = c, including -0 -> 0x8
        assert Q.e2m1_encode(np.array([float(val)]))[0] == c


def test_e8m0_and_element_golden():
    lines = read_golden("e8m0_examples.txt")
    for ln in lines[:6]:
        a, e, byte = [p.strip() for p in ln.split("|")]
        assert Q.e8m0_exponent(np.array([float(a)]))[0] == int(e)
        assert int(e) + 127 == int(byte)
    for ln in lines[6:]:
        v, code = [p.strip() for p in ln.split("|")]
        assert Q.e2m1_encode(np.array([float(v)]))[0] == int(code, 16)


def test_mx_roundtrip_and_error():
    rng = np.random.default_rng(23)
    v = (rng.standard_normal((32, 256)) * np.exp(rng.uniform(-6, 6, size=(32, 1)))).astype(np.float32)
    codes, sb, _, _ = Q.quant_mx(v)
    deq = Q.mx_dequant(codes, sb)
    vb = v.reshape(32, 8, 32).astype(np.float64)
    db = deq.reshape(32, 8, 32)
    e = sb.astype(np.int64) - 127
    a = np.abs(vb).max(axis=-1)
    # a lies in [4, 8) 2^e; grid spacing below 4 2^e is at most 2^e, above it 2 2^e
    assert np.all(a >= 4.0 * np.exp2(e)) and np.all(a < 8.0 * np.exp2(e))
    err = np.abs(vb - db)
    inner = np.abs(vb) <= 6.0 * np.exp2(e)[..., None]
    assert np.all(err[inner] <= (np.exp2(e)[..., None] * np.ones_like(vb))[inner] + 0)
    # dequantized grid points re-encode to themselves
    c2, sb2, _, _ = Q.quant_mx(deq.astype(np.float32))
    np.testing.assert_array_equal(Q.mx_dequant(c2, sb2), deq)


def test_nibble_pack_roundtrip():
    c = np.arange(16, dtype=np.uint8)
    np.testing.assert_array_equal(Q.unpack_nibbles(Q.pack_nibbles(c[None]))[0], c)
    assert Q.pack_nibbles(np.array([[0x3, 0xC]]))[0, 0] == 0xC3


# ---- percentile scale (CentriQ Sec. 4.2 "Scale and grid", App. B.3 Table 3)

def test_normal_quantile_against_scipy():
    stats = pytest.importorskip("scipy.stats")
    z = Q.std_normal_upper_quantile(Q.PCTL_TAIL)
    assert abs(z - stats.norm.isf(0.00025)) <= 2e-15 * z
    assert abs(z - stats.norm.ppf(0.99975)) <= 1e-12 * z
    for tail in (0.5, 0.1, 1e-3, 1e-6):
        assert abs(Q.std_normal_upper_quantile(tail) - stats.norm.isf(tail)) <= 1e-14 * max(1.0, stats.norm.isf(tail))


@pytest.mark.parametrize("n", [16, 100, 1920, 3072, 4096, 5000])
def test_percentile_is_the_linear_empirical_quantile(n):
    # numpy's "linear" method (Hyndman-Fan type 7) is an independent
    # implementation of the same interpolated order statistic
    rng = np.random.default_rng(n)
    v = (rng.standard_normal((5, n)) * rng.uniform(0.1, 10, size=(5, 1))).astype(np.float32)
    r = Q.pctl_range(v).astype(np.float64)
    z = Q.std_normal_upper_quantile(Q.PCTL_TAIL)
    q_np = np.quantile(np.abs(v).astype(np.float64), Q.PCTL_RHO, axis=-1, method="linear")
    want = (q_np * Q.PCTL_GAMMA / z).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(r - want) <= np.spacing(want.astype(np.float32)).astype(np.float64))


def test_percentile_constant_row_and_spread_of_gaussian_rows():
    z = Q.std_normal_upper_quantile(Q.PCTL_TAIL)
    c = np.full((1, 3072), -0.75, dtype=np.float32)
    assert Q.pctl_range(c)[0] == np.float32(0.75 * Q.PCTL_GAMMA / z)
    rng = np.random.default_rng(3)
    sig = np.array([0.01, 1.0, 300.0])
    v = (rng.standard_normal((3, 1 << 17)) * sig[:, None]).astype(np.float32)
    sig_hat = Q.pctl_range(v).astype(np.float64) / Q.PCTL_GAMMA
    assert np.all(np.abs(sig_hat / sig - 1) < 0.05)


def test_gamma_star_minimizes_4bit_gaussian_error():
    # the pages choose gamma* as the minimizer of clipping plus rounding error
    # of a 4-bit grid for Gaussian input: it beats clips 15% tighter and wider
    rng = np.random.default_rng(11)
    v = rng.standard_normal((1, 1 << 21)).astype(np.float32)

    def mse(gamma):
        r = Q.pctl_range(v, gamma=gamma)
        alpha, inv = Q.absmax_scale(r, 7)
        q, _ = Q.round_codes(v, inv[..., None], 7)
        return float(np.mean((alpha[..., None].astype(np.float64) * q - v) ** 2))

    e0 = mse(Q.PCTL_GAMMA)
    assert e0 < mse(0.85 * Q.PCTL_GAMMA) and e0 < mse(1.15 * Q.PCTL_GAMMA)


@pytest.mark.parametrize("qmax", [7, 31, 127])
def test_percentile_codes_clip_beyond_the_range(qmax):
    rng = np.random.default_rng(qmax)
    v = rng.standard_normal((8, 1024)).astype(np.float32)
    v[:, 7] = 40.0  # far beyond the range: clipped
    q, alpha, flag = Q.quant_token_pctl(v, qmax)
    r = Q.pctl_range(v)
    assert np.all(q[:, 7] == qmax)
    assert np.all(np.abs(q) <= qmax)
    assert np.allclose(alpha, r / np.float32(qmax), rtol=2 ** -23)
    inside = np.abs(v) <= 0.9 * r[:, None]
    err = np.abs(alpha[:, None].astype(np.float64) * q - v)
    assert np.all(err[inside] <= 0.5 * alpha.astype(np.float64)[:, None].repeat(1024, 1)[inside] * (1 + 1e-6))
