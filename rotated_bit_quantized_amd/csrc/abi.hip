// C-ABI entry points of liboq: argument validation and kernel dispatch.
//
// Every call validates all of its arguments before anything is enqueued and
// returns an OQ_ERR_* code on the first violation (model card
// FLUX.1-schnell-OrbitQuant-W4A4, "Limitations": the fused runtime fails
// loudly rather than falling back).  Launch failures reported by the HIP
// runtime become OQ_ERR_HIP.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "oq_internal.h"

namespace oq {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

namespace {

inline bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return OQ_OK;
  return fail(OQ_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Validates a bf16 activation matrix [M][ldx] of row width d.
int check_x(const char *fn, const uint16_t *x, int64_t M, int d, int64_t ldx) {
  if (M < 0) return fail(OQ_ERR_INVALID_ARG, "%s: M must be >= 0 (got %lld)", fn, (long long)M);
  if (M > 0 && !x) return fail(OQ_ERR_INVALID_ARG, "%s: x is NULL", fn);
  if (d < 16 || d > 16384 || d % 16)
    return fail(OQ_ERR_UNSUPPORTED, "%s: width d=%d must be a multiple of 16 in [16, 16384]", fn, d);
  if (ldx < d) return fail(OQ_ERR_INVALID_ARG, "%s: ldx=%lld < d=%d", fn, (long long)ldx, d);
  if (!al16(x) || (ldx * 2) % 16) return fail(OQ_ERR_ALIGNMENT, "%s: x rows must be 16-byte aligned", fn);
  return OQ_OK;
}

// Fills RotArgs from an RPBH descriptor (or identity when rot == NULL).
int rot_args(const char *fn, const oq_rot *rot, int d, RotArgs *ra) {
  ra->rounds = 0;
  ra->block = 16;
  ra->perm = nullptr;
  ra->signs = nullptr;
  ra->c_h = 1.0f;
  ra->kron_m = 0;
  if (!rot) return OQ_OK;
  if (rot->kind == OQ_ROT_KRON) {
    const int m = rot->rounds, b = rot->block;
    if (rot->d != d) return fail(OQ_ERR_INVALID_ARG, "%s: rot->d=%d differs from d=%d", fn, rot->d, d);
    if (m != 1 && m != 12 && m != 36 && m != 44)
      return fail(OQ_ERR_UNSUPPORTED, "%s: Paley order m=%d must be 1, 12, 36 or 44", fn, m);
    if (!is_pow2(b) || b < 16) return fail(OQ_ERR_UNSUPPORTED, "%s: block=%d must be a power of two >= 16", fn, b);
    if ((int64_t)m * b < d || (int64_t)m * b > 16384)
      return fail(OQ_ERR_UNSUPPORTED, "%s: padded width m*block=%lld must lie in [d, 16384]", fn, (long long)m * b);
    ra->rounds = 1;
    ra->block = b;
    ra->kron_m = m;
    ra->c_h = (float)(1.0 / std::sqrt((double)m * (double)b));
    return OQ_OK;
  }
  if (rot->kind != OQ_ROT_RPBH) return fail(OQ_ERR_INVALID_ARG, "%s: expected an RPBH rotation", fn);
  if (rot->d != d) return fail(OQ_ERR_INVALID_ARG, "%s: rot->d=%d differs from d=%d", fn, rot->d, d);
  if (!is_pow2(rot->block) || rot->block < 32 || rot->block > 1024)
    return fail(OQ_ERR_UNSUPPORTED, "%s: block=%d must be a power of two in [32, 1024]", fn, rot->block);
  if (d % rot->block) return fail(OQ_ERR_INVALID_ARG, "%s: d=%d not a multiple of block=%d", fn, d, rot->block);
  if (rot->rounds < 1 || rot->rounds > 2) return fail(OQ_ERR_UNSUPPORTED, "%s: rounds=%d must be 1 or 2", fn, rot->rounds);
  if (!rot->perm || !rot->signs) return fail(OQ_ERR_INVALID_ARG, "%s: perm/signs are NULL", fn);
  ra->rounds = rot->rounds;
  ra->block = rot->block;
  ra->perm = rot->perm;
  ra->signs = rot->signs;
  ra->c_h = (float)(1.0 / std::sqrt((double)rot->block));
  return OQ_OK;
}

int check_dense(const char *fn, const oq_rot *rot, int d) {
  if (rot->d != d) return fail(OQ_ERR_INVALID_ARG, "%s: rot->d=%d differs from d=%d", fn, rot->d, d);
  if (d % 32) return fail(OQ_ERR_INVALID_ARG, "%s: d=%d must be a multiple of 32", fn, d);
  if (!rot->mats) return fail(OQ_ERR_INVALID_ARG, "%s: transform matrices are NULL", fn);
  if (reinterpret_cast<uintptr_t>(rot->mats) & 15)
    return fail(OQ_ERR_ALIGNMENT, "%s: rot->mats must be 16-byte aligned", fn);
  return OQ_OK;
}

int qmax_of(int afmt) { return afmt == OQ_A8 ? 127 : afmt == OQ_A6 ? 31 : 7; }

// x with Phi(-x) = tail (the standard normal upper quantile), by bisection on
// erfc(x / sqrt 2) / 2 = tail until the bracket cannot shrink
double upper_normal_quantile(double tail) {
  double lo = 0.0, hi = 40.0;
  for (;;) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (0.5 * std::erfc(mid / std::sqrt(2.0)) > tail)
      lo = mid;
    else
      hi = mid;
  }
  return hi;
}

// CentriQ Sec. 4.2 "Scale and grid", App. B.3 Table 3: rho = 0.9995, gamma* =
// 2.5591; the rho-quantile of d magnitudes interpolates between the order
// statistics k = floor(rho (d - 1)) and k + 1 (ascending), i.e. the
// (d - k)-th and (d - k - 1)-th largest.
int pctl_setup(const char *fn, int afmt, int d, PctlArgs *pa) {
  const int base = afmt & ~OQ_TILED;
  if (base != OQ_A8 && base != OQ_A6 && base != OQ_A4)
    return fail(OQ_ERR_UNSUPPORTED, "%s: OQ_SCALE_PCTL applies to integer activation codes", fn);
  if (!rpbh_wave_supported(d))
    return fail(OQ_ERR_UNSUPPORTED, "%s: OQ_SCALE_PCTL needs d %% 16 == 0 and 16 <= d <= 4096 (d=%d)", fn, d);
  const double h = 0.9995 * (double)(d - 1);
  const double k = std::floor(h);
  pa->rank = d - (int)k;
  pa->frac = h - k;
  pa->gamma = 2.5591;
  pa->z = upper_normal_quantile(0.00025);
  if (pa->rank < 2 || pa->rank > 4) return fail(OQ_ERR_UNSUPPORTED, "%s: percentile rank %d", fn, pa->rank);
  return OQ_OK;
}

// float64 -> float16 bits, round to nearest even (host)
uint16_t f64_to_f16_rne(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  const double a = std::fabs(x);
  if (a == 0.0) return sign;
  if (!(a < 65520.0)) return sign | 0x7C00u;  // rounds to infinity (or NaN input)
  int e;
  (void)std::frexp(a, &e);                       // a = m 2^e, m in [0.5, 1)
  int E = e - 1;                                 // a = 1.f 2^E
  const int qexp = (E < -14 ? -14 : E) - 10;     // value of the last float16 bit
  const double r = std::nearbyint(std::ldexp(a, -qexp));  // exact scaling, RNE (default mode)
  uint32_t bits;
  if (E < -14) {
    bits = (uint32_t)r;  // subnormal; r == 1024 is the smallest normal
  } else {
    double rr = r;
    if (rr >= 2048.0) {
      rr *= 0.5;
      ++E;
    }
    if (E > 15) return sign | 0x7C00u;
    bits = ((uint32_t)(E + 15) << 10) | ((uint32_t)rr - 1024u);
  }
  return sign | (uint16_t)bits;
}

float f16_to_f32(uint16_t h) {
  const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v;
  if (e == 0) v = std::ldexp((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((float)(m | 0x400), (int)e - 25);
  return (h & 0x8000) ? -v : v;
}

int check_lm_bits(const char *fn, int bits) {
  if (bits < 1 || bits > 8) return fail(OQ_ERR_UNSUPPORTED, "%s: bits=%d must be in [1, 8]", fn, bits);
  return OQ_OK;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct LinearWs {
  size_t codes, scale, mean, total;
  int64_t ldc;
};

LinearWs linear_ws(int64_t M, int K, int afmt) {
  LinearWs w;
  const int base_fmt = afmt & ~OQ_TILED;
  w.ldc = (base_fmt == OQ_A8 || base_fmt == OQ_A6) ? K : K / 2;
  w.ldc = (w.ldc + 15) & ~(int64_t)15;
  w.codes = 0;
  size_t code_bytes = (afmt & OQ_TILED) ? (size_t)(base_fmt == OQ_A6 ? 2 : 1) * tiled_bytes(M, K)
                                        : (size_t)M * w.ldc;
  size_t sbytes = base_fmt == OQ_MXFP4 ? (size_t)M * (K / 32) : (size_t)M * 4;
  if (afmt == (OQ_MXFP4 | OQ_TILED)) {
    code_bytes = (size_t)tiled_mx_bytes(M, K);
    sbytes = code_bytes / 16;
  }
  w.scale = align_up(code_bytes);
  w.mean = align_up(w.scale + sbytes);
  w.total = align_up(w.mean + (size_t)M * 4);
  return w;
}

int check_gemm_common(const char *fn, const void *qa, int64_t lda_bytes, int64_t M, int K, const uint8_t *w,
                      const void *w_scale, int N, const uint16_t *y, int64_t ldy, int64_t min_lda) {
  if (M < 0 || N < 0) return fail(OQ_ERR_INVALID_ARG, "%s: negative M or N", fn);
  if (K <= 0 || K % 64) return fail(OQ_ERR_UNSUPPORTED, "%s: K=%d must be a positive multiple of 64", fn, K);
  if (M == 0 || N == 0) return OQ_OK;
  if (!qa || !w || !w_scale || !y) return fail(OQ_ERR_INVALID_ARG, "%s: NULL operand", fn);
  if (lda_bytes < min_lda) return fail(OQ_ERR_INVALID_ARG, "%s: lda too small", fn);
  if (!al16(qa) || lda_bytes % 16 || !al16(w)) return fail(OQ_ERR_ALIGNMENT, "%s: codes must be 16-byte aligned rows", fn);
  if (ldy < N) return fail(OQ_ERR_INVALID_ARG, "%s: ldy=%lld < N=%d", fn, (long long)ldy, N);
  if (reinterpret_cast<uintptr_t>(y) & 1) return fail(OQ_ERR_ALIGNMENT, "%s: y misaligned", fn);
  return OQ_OK;
}

int check_int_epilogue(const char *fn, int K, int group, const float *mean, const float *w1) {
  if (group < 32 || group % 32 || K % group)
    return fail(OQ_ERR_UNSUPPORTED, "%s: group=%d must be a multiple of 32 dividing K=%d", fn, group, K);
  if ((mean == nullptr) != (w1 == nullptr)) return fail(OQ_ERR_INVALID_ARG, "%s: mean and w1 must be given together", fn);
  return OQ_OK;
}

}  // namespace
}  // namespace oq

using namespace oq;

extern "C" {

const char *oq_last_error(void) { return g_err; }

int oq_center(const uint16_t *x, int64_t M, int32_t d, int64_t ldx, float *xc, int64_t ldxc, float *mean,
              hipStream_t stream) {
  int rc = check_x("oq_center", x, M, d, ldx);
  if (rc) return rc;
  if (M > 0 && !mean) return fail(OQ_ERR_INVALID_ARG, "oq_center: mean is NULL");
  if (xc && (ldxc < d || !al16(xc) || (ldxc * 4) % 16)) return fail(OQ_ERR_ALIGNMENT, "oq_center: bad xc layout");
  g_err[0] = 0;
  RotArgs ra;
  rot_args("oq_center", nullptr, d, &ra);
  return hip_status(launch_rpbh_quant(x, M, d, ldx, ra, 1, mean, OUT_F32, 0, xc, ldxc * 4, nullptr, stream),
                    "oq_center");
}

int oq_rotate(const oq_rot *rot, const uint16_t *x, int64_t M, int64_t ldx, int center, float *mean, float *y,
              int64_t ldy, hipStream_t stream) {
  if (!rot) return fail(OQ_ERR_INVALID_ARG, "oq_rotate: rot is NULL");
  const int d = rot->d;
  int rc = check_x("oq_rotate", x, M, d, ldx);
  if (rc) return rc;
  if (M > 0 && !y) return fail(OQ_ERR_INVALID_ARG, "oq_rotate: y is NULL");
  const int dy = rot->kind == OQ_ROT_KRON ? rot->rounds * rot->block : d;
  if (ldy < dy || !al16(y) || (ldy * 4) % 16) return fail(OQ_ERR_ALIGNMENT, "oq_rotate: bad y layout");
  if (center && !mean) return fail(OQ_ERR_INVALID_ARG, "oq_rotate: centering needs mean");
  if (rot->kind == OQ_ROT_DENSE32) {
    if (center) return fail(OQ_ERR_UNSUPPORTED, "oq_rotate: centering with a DENSE32 rotation");
    rc = check_dense("oq_rotate", rot, d);
    if (rc) return rc;
    g_err[0] = 0;
    return hip_status(launch_dense32(x, M, d, ldx, rot->mats, 0, y, ldy * 4, nullptr, stream), "oq_rotate");
  }
  RotArgs ra;
  rc = rot_args("oq_rotate", rot, d, &ra);
  if (rc) return rc;
  g_err[0] = 0;
  return hip_status(launch_rpbh_quant(x, M, d, ldx, ra, center ? 1 : 0, mean, OUT_F32, 0, y, ldy * 4, nullptr, stream),
                    "oq_rotate");
}

int oq_quant_act(const uint16_t *x, int64_t M, int32_t d, int64_t ldx, const oq_rot *rot, int center, int afmt,
                 void *codes, int64_t ldc_bytes, float *scale, uint8_t *e8m0, float *mean, hipStream_t stream) {
  int rc = check_x("oq_quant_act", x, M, d, ldx);
  if (rc) return rc;
  PctlArgs pa;
  const PctlArgs *pp = nullptr;
  if (afmt & OQ_SCALE_PCTL) {
    afmt &= ~OQ_SCALE_PCTL;
    rc = pctl_setup("oq_quant_act", afmt, d, &pa);
    if (rc) return rc;
    pp = &pa;
  }
  if (M > 0 && !codes) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: codes is NULL");
  if (!al16(codes) || (!(afmt & OQ_TILED) && ldc_bytes % 16))
    return fail(OQ_ERR_ALIGNMENT, "oq_quant_act: code rows must be 16-byte aligned");
  if (afmt == (OQ_MXFP4 | OQ_TILED)) {
    if (!rot || rot->kind != OQ_ROT_DENSE32)
      return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: MXFP4 activations need a DENSE32 rotation");
    if (center) return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: centering is not defined for MXFP4 here");
    if (d % 128) return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: tiled MXFP4 needs d %% 128 == 0 (d=%d)", d);
    if (M > 0 && !e8m0) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: e8m0 is NULL");
    if (reinterpret_cast<uintptr_t>(e8m0) & 3) return fail(OQ_ERR_ALIGNMENT, "oq_quant_act: e8m0 must be 4-byte aligned");
    if (scale) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: scale must be NULL for MXFP4");
    rc = check_dense("oq_quant_act", rot, d);
    if (rc) return rc;
    g_err[0] = 0;
    return hip_status(launch_dense32(x, M, d, ldx, rot->mats, 2, codes, 0, e8m0, stream), "oq_quant_act");
  }
  if (afmt == OQ_MXFP4) {
    if (!rot || rot->kind != OQ_ROT_DENSE32)
      return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: MXFP4 activations need a DENSE32 rotation");
    if (center) return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: centering is not defined for MXFP4 here");
    if (ldc_bytes < d / 2) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: ldc_bytes < d/2");
    if (M > 0 && !e8m0) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: e8m0 is NULL");
    if (scale) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: scale must be NULL for MXFP4");
    rc = check_dense("oq_quant_act", rot, d);
    if (rc) return rc;
    g_err[0] = 0;
    return hip_status(launch_dense32(x, M, d, ldx, rot->mats, 1, codes, ldc_bytes, e8m0, stream), "oq_quant_act");
  }
  const bool tiled = (afmt & OQ_TILED) != 0;
  const int base_fmt = afmt & ~OQ_TILED;
  if (tiled) {
    if (base_fmt != OQ_A4 && base_fmt != OQ_A6)
      return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: the tiled layout exists for OQ_A4, OQ_A6 and OQ_MXFP4");
    if (e8m0) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: e8m0 must be NULL for integer codes");
    if (M > 0 && !scale) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: scale is NULL");
    if (center && !mean) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: centering needs mean");
    RotArgs ra;
    rc = rot_args("oq_quant_act", rot, d, &ra);
    if (rc) return rc;
    if (rot_out_width(ra, d) % 64)
      return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: tiled codes need a width multiple of 64 (%d)", rot_out_width(ra, d));
    if (ra.kron_m && pp) return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: OQ_SCALE_PCTL with the Kronecker rotation");
    g_err[0] = 0;
    return hip_status(launch_rpbh_quant(x, M, d, ldx, ra, center ? 1 : 0, mean,
                                        base_fmt == OQ_A4 ? OUT_FP6 : OUT_FP6X2, qmax_of(base_fmt), codes, 0,
                                        scale, stream, pp),
                      "oq_quant_act");
  }
  if (afmt != OQ_A8 && afmt != OQ_A6 && afmt != OQ_A4)
    return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: unknown afmt %d", afmt);
  if (e8m0) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: e8m0 must be NULL for integer codes");
  if (M > 0 && !scale) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: scale is NULL");
  if (center && !mean) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: centering needs mean");
  RotArgs ra;
  rc = rot_args("oq_quant_act", rot, d, &ra);
  if (rc) return rc;
  const int dq = rot_out_width(ra, d);
  if (ldc_bytes < (afmt == OQ_A4 ? dq / 2 : dq)) return fail(OQ_ERR_INVALID_ARG, "oq_quant_act: ldc_bytes too small");
  if (ra.kron_m && pp) return fail(OQ_ERR_UNSUPPORTED, "oq_quant_act: OQ_SCALE_PCTL with the Kronecker rotation");
  g_err[0] = 0;
  return hip_status(launch_rpbh_quant(x, M, d, ldx, ra, center ? 1 : 0, mean, afmt == OQ_A4 ? OUT_I4 : OUT_I8,
                                      qmax_of(afmt), codes, ldc_bytes, scale, stream, pp),
                    "oq_quant_act");
}

int oq_quant_weight(const float *w, int32_t N, int32_t K, int64_t ldw, const oq_rot *rot, int wfmt, int32_t group,
                    uint8_t *codes, void *scales, float *w1, hipStream_t stream) {
  if (N < 0) return fail(OQ_ERR_INVALID_ARG, "oq_quant_weight: N < 0");
  if (K < 32 || K > 16384 || K % 32) return fail(OQ_ERR_UNSUPPORTED, "oq_quant_weight: K=%d must be a multiple of 32 in [32, 16384]", K);
  if (ldw < K) return fail(OQ_ERR_INVALID_ARG, "oq_quant_weight: ldw < K");
  if (N > 0 && (!w || !codes || !scales)) return fail(OQ_ERR_INVALID_ARG, "oq_quant_weight: NULL pointer");
  if (!al16(w) || (ldw * 4) % 16 || !al16(codes)) return fail(OQ_ERR_ALIGNMENT, "oq_quant_weight: misaligned");
  if (wfmt == OQ_W_MXFP4) {
    if (!rot || rot->kind != OQ_ROT_DENSE32) return fail(OQ_ERR_UNSUPPORTED, "oq_quant_weight: MXFP4 weights need DENSE32");
    if (w1) return fail(OQ_ERR_UNSUPPORTED, "oq_quant_weight: w1 is produced for OQ_W4 only");
    int rc = check_dense("oq_quant_weight", rot, K);
    if (rc) return rc;
    g_err[0] = 0;
    return hip_status(launch_weight_dense32(w, N, K, ldw, rot->mats, codes, (uint8_t *)scales, nullptr, stream),
                      "oq_quant_weight");
  }
  if (wfmt != OQ_W4) return fail(OQ_ERR_INVALID_ARG, "oq_quant_weight: unknown wfmt %d", wfmt);
  RotArgs ra;
  int rc = rot_args("oq_quant_weight", rot, K, &ra);
  if (rc) return rc;
  const int Kq = rot_out_width(ra, K);
  if (!is_pow2(group) || group < 32 || group > 1024 || Kq % group)
    return fail(OQ_ERR_UNSUPPORTED, "oq_quant_weight: group=%d must be a power of two in [32, 1024] dividing %d", group, Kq);
  g_err[0] = 0;
  return hip_status(launch_weight_rpbh(w, N, K, ldw, ra, group, codes, (float *)scales, w1, stream), "oq_quant_weight");
}

int oq_gemm_w4a8(const int8_t *qa, int64_t lda, const float *a_scale, int64_t M, int32_t K, const uint8_t *w,
                 const float *w_scale, int32_t N, int32_t group, const float *mean, const float *w1,
                 const float *bias, uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_gemm_common("oq_gemm_w4a8", qa, lda, M, K, w, w_scale, N, y, ldy, K);
  if (rc) return rc;
  rc = check_int_epilogue("oq_gemm_w4a8", K, group, mean, w1);
  if (rc) return rc;
  if (M > 0 && !a_scale) return fail(OQ_ERR_INVALID_ARG, "oq_gemm_w4a8: a_scale is NULL");
  if (ws && !al16(ws)) return fail(OQ_ERR_ALIGNMENT, "oq_gemm_w4a8: workspace must be 16-byte aligned");
  g_err[0] = 0;
  return hip_status(launch_gemm_int(qa, lda, 0, a_scale, M, K, w, w_scale, N, group, mean, w1, bias, y, ldy, stream,
                                    ws, ws ? ws_bytes : 0),
                    "oq_gemm_w4a8");
}

int oq_gemm_w4a4(int afmt, const uint8_t *qa, int64_t lda_bytes, const void *a_scale, int64_t M, int32_t K,
                 const uint8_t *w, const void *w_scale, int32_t N, int32_t group, const float *mean, const float *w1,
                 const float *bias, uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (afmt == (OQ_MXFP4 | OQ_TILED)) {
    int rc = check_gemm_common("oq_gemm_w4a4", qa, 16, M, K, w, w_scale, N, y, ldy, 0);
    if (rc) return rc;
    if (K % 128) return fail(OQ_ERR_UNSUPPORTED, "oq_gemm_w4a4: tiled MXFP4 needs K %% 128 == 0 (K=%d)", K);
    if (group != 32) return fail(OQ_ERR_INVALID_ARG, "oq_gemm_w4a4: MXFP4 blocks are 32 (group=%d)", group);
    if (mean || w1) return fail(OQ_ERR_UNSUPPORTED, "oq_gemm_w4a4: rank-1 restore is not defined for MXFP4 here");
    if (M > 0 && N > 0 && !a_scale) return fail(OQ_ERR_INVALID_ARG, "oq_gemm_w4a4: a_scale is NULL");
    if ((reinterpret_cast<uintptr_t>(a_scale) | reinterpret_cast<uintptr_t>(w_scale)) & 3)
      return fail(OQ_ERR_ALIGNMENT, "oq_gemm_w4a4: tiled E8M0 scale words must be 4-byte aligned");
    g_err[0] = 0;
    return hip_status(launch_gemm_mx(1, qa, 0, (const uint8_t *)a_scale, M, K, w, (const uint8_t *)w_scale, N, bias,
                                     y, ldy, stream),
                      "oq_gemm_w4a4");
  }
  if (afmt & OQ_TILED) {
    const int base_fmt = afmt & ~OQ_TILED;
    int rc = check_gemm_common("oq_gemm_w4a4", qa, 16, M, K, w, w_scale, N, y, ldy, 0);
    if (rc) return rc;
    if (base_fmt != OQ_A4 && base_fmt != OQ_A6)
      return fail(OQ_ERR_UNSUPPORTED, "oq_gemm_w4a4: tiled operands exist for OQ_A4, OQ_A6 and OQ_MXFP4");
    if (group != 64) return fail(OQ_ERR_UNSUPPORTED, "oq_gemm_w4a4: tiled GEMM needs group 64 (got %d)", group);
    if (!fp6_offsets_fit(M, N, K))
      return fail(OQ_ERR_UNSUPPORTED, "oq_gemm_w4a4: a tiled operand plane exceeds 4 GiB (split M or N)");
    rc = check_int_epilogue("oq_gemm_w4a4", K, group, mean, w1);
    if (rc) return rc;
    if (M > 0 && N > 0 && !a_scale) return fail(OQ_ERR_INVALID_ARG, "oq_gemm_w4a4: a_scale is NULL");
    g_err[0] = 0;
    return hip_status(launch_gemm_fp6(qa, base_fmt == OQ_A6 ? 2 : 1, (const float *)a_scale, M, K, w,
                                      (const float *)w_scale, N, mean, w1, bias, y, ldy, stream),
                      "oq_gemm_w4a4");
  }
  int rc = check_gemm_common("oq_gemm_w4a4", qa, lda_bytes, M, K, w, w_scale, N, y, ldy, K / 2);
  if (rc) return rc;
  if (M > 0 && N > 0 && !a_scale) return fail(OQ_ERR_INVALID_ARG, "oq_gemm_w4a4: a_scale is NULL");
  if (afmt == OQ_MXFP4) {
    if (group != 32) return fail(OQ_ERR_INVALID_ARG, "oq_gemm_w4a4: MXFP4 blocks are 32 (group=%d)", group);
    if (mean || w1) return fail(OQ_ERR_UNSUPPORTED, "oq_gemm_w4a4: rank-1 restore is not defined for MXFP4 here");
    g_err[0] = 0;
    return hip_status(launch_gemm_mx(0, qa, lda_bytes, (const uint8_t *)a_scale, M, K, w, (const uint8_t *)w_scale, N,
                                     bias, y, ldy, stream),
                      "oq_gemm_w4a4");
  }
  if (afmt != OQ_A4) return fail(OQ_ERR_INVALID_ARG, "oq_gemm_w4a4: afmt must be OQ_A4 or OQ_MXFP4");
  rc = check_int_epilogue("oq_gemm_w4a4", K, group, mean, w1);
  if (rc) return rc;
  g_err[0] = 0;
  return hip_status(launch_gemm_int(qa, lda_bytes, 1, (const float *)a_scale, M, K, w, (const float *)w_scale, N,
                                    group, mean, w1, bias, y, ldy, stream),
                    "oq_gemm_w4a4");
}

size_t oq_tiled_bytes(int64_t rows, int32_t K) {
  if (rows < 0 || K <= 0) return 0;
  return (size_t)tiled_bytes(rows, K);
}

int oq_prepack_w4(const uint8_t *w, const float *w_scale, int32_t N, int32_t K, int32_t group, uint8_t *w_tiled,
                  float *w_scale_t, hipStream_t stream) {
  if (N < 0) return fail(OQ_ERR_INVALID_ARG, "oq_prepack_w4: N < 0");
  if (K <= 0 || K % 64) return fail(OQ_ERR_UNSUPPORTED, "oq_prepack_w4: K=%d must be a positive multiple of 64", K);
  if (group != 64) return fail(OQ_ERR_UNSUPPORTED, "oq_prepack_w4: group must be 64 (got %d)", group);
  if (N > 0 && (!w || !w_scale || !w_tiled || !w_scale_t)) return fail(OQ_ERR_INVALID_ARG, "oq_prepack_w4: NULL pointer");
  if (!al16(w) || !al16(w_tiled)) return fail(OQ_ERR_ALIGNMENT, "oq_prepack_w4: misaligned");
  g_err[0] = 0;
  return hip_status(launch_prepack_w4(w, w_scale, N, K, w_tiled, w_scale_t, stream), "oq_prepack_w4");
}

size_t oq_tiled_mx_bytes(int64_t rows, int32_t K) {
  if (rows < 0 || K <= 0) return 0;
  return (size_t)tiled_mx_bytes(rows, K);
}

int oq_prepack_mx(const uint8_t *w, const uint8_t *w_e8m0, int32_t N, int32_t K, uint8_t *w_tiled,
                  uint8_t *w_e8m0_tiled, hipStream_t stream) {
  if (N < 0) return fail(OQ_ERR_INVALID_ARG, "oq_prepack_mx: N < 0");
  if (K <= 0 || K % 128) return fail(OQ_ERR_UNSUPPORTED, "oq_prepack_mx: K=%d must be a positive multiple of 128", K);
  if (N > 0 && (!w || !w_e8m0 || !w_tiled || !w_e8m0_tiled)) return fail(OQ_ERR_INVALID_ARG, "oq_prepack_mx: NULL pointer");
  if (!al16(w) || !al16(w_tiled) || (reinterpret_cast<uintptr_t>(w_e8m0_tiled) & 3))
    return fail(OQ_ERR_ALIGNMENT, "oq_prepack_mx: misaligned");
  g_err[0] = 0;
  return hip_status(launch_prepack_mx(w, w_e8m0, N, K, w_tiled, w_e8m0_tiled, stream), "oq_prepack_mx");
}

size_t oq_workspace_bytes(int op, int64_t M, int32_t K, int32_t N, int afmt) {
  if (M < 0 || K <= 0) return 0;
  if (op == OQ_OP_GEMM_LM) return (afmt & OQ_TILED) ? 0 : (size_t)tiled_f16_bytes(M, K);
  if (op == OQ_OP_GEMM_W4A8) return N > 0 ? int_gemm_split_bytes(M, N, K) : 0;
  if (op != OQ_OP_LINEAR) return 0;
  return linear_ws(M, K, afmt & ~OQ_SCALE_PCTL).total;
}

}  // extern "C"

namespace oq {
namespace {

// The whole layer into a given workspace (validation first, then K1 and the
// GEMM on `stream`); shared by oq_linear_fused and oq_linear_fused_noalloc.
int linear_fused_impl(const char *fn, const uint16_t *x, int64_t M, int32_t K, int64_t ldx, const oq_rot *rot,
                      int center, int afmt, const uint8_t *w, const void *w_scale, int32_t N, int32_t group,
                      const float *w1, const float *bias, uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes,
                      hipStream_t stream) {
  int rc = check_x(fn, x, M, K, ldx);
  if (rc) return rc;
  if (rot && rot->kind == OQ_ROT_KRON)
    return fail(OQ_ERR_UNSUPPORTED, "%s: the Kronecker rotation pads the width; call oq_quant_act and a GEMM", fn);
  PctlArgs pa;
  const PctlArgs *pp = nullptr;
  if (afmt & OQ_SCALE_PCTL) {
    afmt &= ~OQ_SCALE_PCTL;
    rc = pctl_setup(fn, afmt, K, &pa);
    if (rc) return rc;
    pp = &pa;
  }
  if (afmt == (OQ_MXFP4 | OQ_TILED)) {
    if (!rot || rot->kind != OQ_ROT_DENSE32) return fail(OQ_ERR_UNSUPPORTED, "%s: MXFP4 needs a DENSE32 rotation", fn);
    if (center || w1) return fail(OQ_ERR_UNSUPPORTED, "%s: centering is not defined for MXFP4 here", fn);
    if (group != 32) return fail(OQ_ERR_INVALID_ARG, "%s: MXFP4 blocks are 32 (group=%d)", fn, group);
    if (K % 128) return fail(OQ_ERR_UNSUPPORTED, "%s: tiled MXFP4 needs K %% 128 == 0", fn);
    const LinearWs L = linear_ws(M, K, afmt);
    if (M > 0 && (!ws || ws_bytes < L.total))
      return fail(OQ_ERR_WORKSPACE, "%s: workspace of %zu bytes required (got %zu)", fn, L.total, ws_bytes);
    if (ws && !al16(ws)) return fail(OQ_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", fn);
    rc = check_gemm_common(fn, x, 16, M, K, w, w_scale, N, y, ldy, 0);
    if (rc) return rc;
    if (reinterpret_cast<uintptr_t>(w_scale) & 3)
      return fail(OQ_ERR_ALIGNMENT, "%s: tiled E8M0 scale words must be 4-byte aligned", fn);
    rc = check_dense(fn, rot, K);
    if (rc) return rc;
    char *wsb = static_cast<char *>(ws);
    uint8_t *codes = reinterpret_cast<uint8_t *>(wsb + L.codes);
    uint8_t *e8 = reinterpret_cast<uint8_t *>(wsb + L.scale);
    g_err[0] = 0;
    rc = hip_status(launch_dense32(x, M, K, ldx, rot->mats, 2, codes, 0, e8, stream), fn);
    if (rc) return rc;
    return hip_status(launch_gemm_mx(1, codes, 0, e8, M, K, w, (const uint8_t *)w_scale, N, bias, y, ldy, stream), fn);
  }
  if (afmt & OQ_TILED) {
    const int base_fmt = afmt & ~OQ_TILED;
    if (base_fmt != OQ_A4 && base_fmt != OQ_A6)
      return fail(OQ_ERR_UNSUPPORTED, "%s: tiled operands exist for OQ_A4, OQ_A6 and OQ_MXFP4", fn);
    if (K % 64) return fail(OQ_ERR_UNSUPPORTED, "%s: tiled operands need K %% 64 == 0", fn);
    if (group != 64) return fail(OQ_ERR_UNSUPPORTED, "%s: tiled GEMM needs group 64 (got %d)", fn, group);
    if (!fp6_offsets_fit(M, N, K)) return fail(OQ_ERR_UNSUPPORTED, "%s: a tiled operand plane exceeds 4 GiB (split M or N)", fn);
    const LinearWs L = linear_ws(M, K, afmt);
    if (M > 0 && (!ws || ws_bytes < L.total))
      return fail(OQ_ERR_WORKSPACE, "%s: workspace of %zu bytes required (got %zu)", fn, L.total, ws_bytes);
    if (ws && !al16(ws)) return fail(OQ_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", fn);
    rc = check_gemm_common(fn, x, 16, M, K, w, w_scale, N, y, ldy, 0);
    if (rc) return rc;
    if (center && !w1) return fail(OQ_ERR_INVALID_ARG, "%s: centering needs w1", fn);
    RotArgs ra;
    rc = rot_args(fn, rot, K, &ra);
    if (rc) return rc;
    char *wsb = static_cast<char *>(ws);
    uint8_t *codes = reinterpret_cast<uint8_t *>(wsb + L.codes);
    float *scale = reinterpret_cast<float *>(wsb + L.scale);
    float *mean = reinterpret_cast<float *>(wsb + L.mean);
    g_err[0] = 0;
    rc = hip_status(launch_rpbh_quant(x, M, K, ldx, ra, center ? 1 : 0, mean, base_fmt == OQ_A4 ? OUT_FP6 : OUT_FP6X2,
                                      qmax_of(base_fmt), codes, 0, scale, stream, pp),
                    fn);
    if (rc) return rc;
    return hip_status(launch_gemm_fp6(codes, base_fmt == OQ_A6 ? 2 : 1, scale, M, K, w, (const float *)w_scale, N,
                                      center ? mean : nullptr, center ? w1 : nullptr, bias, y, ldy, stream),
                      fn);
  }
  if (afmt != OQ_A8 && afmt != OQ_A6 && afmt != OQ_A4 && afmt != OQ_MXFP4)
    return fail(OQ_ERR_INVALID_ARG, "%s: unknown afmt %d", fn, afmt);
  const LinearWs L = linear_ws(M, K, afmt);
  if (M > 0 && (!ws || ws_bytes < L.total))
    return fail(OQ_ERR_WORKSPACE, "%s: workspace of %zu bytes required (got %zu)", fn, L.total, ws_bytes);
  if (ws && !al16(ws)) return fail(OQ_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", fn);
  rc = check_gemm_common(fn, x, L.ldc, M, K, w, w_scale, N, y, ldy, 0);
  if (rc) return rc;
  char *wsb = static_cast<char *>(ws);
  uint8_t *codes = reinterpret_cast<uint8_t *>(wsb + L.codes);
  if (afmt == OQ_MXFP4) {
    if (!rot || rot->kind != OQ_ROT_DENSE32) return fail(OQ_ERR_UNSUPPORTED, "%s: MXFP4 needs a DENSE32 rotation", fn);
    if (center || w1) return fail(OQ_ERR_UNSUPPORTED, "%s: centering is not defined for MXFP4 here", fn);
    if (group != 32) return fail(OQ_ERR_INVALID_ARG, "%s: MXFP4 blocks are 32 (group=%d)", fn, group);
    rc = check_dense(fn, rot, K);
    if (rc) return rc;
    uint8_t *e8 = reinterpret_cast<uint8_t *>(wsb + L.scale);
    g_err[0] = 0;
    rc = hip_status(launch_dense32(x, M, K, ldx, rot->mats, 1, codes, L.ldc, e8, stream), fn);
    if (rc) return rc;
    return hip_status(launch_gemm_mx(0, codes, L.ldc, e8, M, K, w, (const uint8_t *)w_scale, N, bias, y, ldy, stream), fn);
  }
  rc = check_int_epilogue(fn, K, group, center ? w1 : nullptr, center ? w1 : nullptr);
  if (rc) return rc;
  if (center && !w1) return fail(OQ_ERR_INVALID_ARG, "%s: centering needs w1", fn);
  RotArgs ra;
  rc = rot_args(fn, rot, K, &ra);
  if (rc) return rc;
  float *scale = reinterpret_cast<float *>(wsb + L.scale);
  float *mean = reinterpret_cast<float *>(wsb + L.mean);
  g_err[0] = 0;
  rc = hip_status(launch_rpbh_quant(x, M, K, ldx, ra, center ? 1 : 0, mean, afmt == OQ_A4 ? OUT_I4 : OUT_I8,
                                    qmax_of(afmt), codes, L.ldc, scale, stream, pp),
                  fn);
  if (rc) return rc;
  return hip_status(launch_gemm_int(codes, L.ldc, afmt == OQ_A4 ? 1 : 0, scale, M, K, w, (const float *)w_scale, N, group,
                                    center ? mean : nullptr, center ? w1 : nullptr, bias, y, ldy, stream),
                    fn);
}


// Scratch of oq_linear_fused_noalloc: one copy per GPU, held by the loaded
// code object until the process ends.  Host code uses the device address that
// hipGetSymbolAddress returns for the current device, never the array's name.
constexpr size_t NOALLOC_BYTES = OQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[NOALLOC_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch, looked up on the first
// call on that device.
int scratch_for_current_device(const char *fn, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= MAX_DEVICES) return fail(OQ_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (!p) return fail(OQ_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OQ_OK;
}

}  // namespace
}  // namespace oq

extern "C" {

int oq_linear_fused(const uint16_t *x, int64_t M, int32_t K, int64_t ldx, const oq_rot *rot, int center, int afmt,
                    const uint8_t *w, const void *w_scale, int32_t N, int32_t group, const float *w1, const float *bias,
                    uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream) {
  return linear_fused_impl("oq_linear_fused", x, M, K, ldx, rot, center, afmt, w, w_scale, N, group, w1, bias, y,
                           ldy, ws, ws_bytes, stream);
}

int oq_linear_fused_noalloc(const uint16_t *x, int64_t M, int32_t K, int64_t ldx, const oq_rot *rot, int center,
                            int afmt, const uint8_t *w, const void *w_scale, int32_t N, int32_t group,
                            const float *w1, const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream) {
  const char *fn = "oq_linear_fused_noalloc";
  if (M < 0 || K <= 0) return fail(OQ_ERR_INVALID_ARG, "%s: bad M or K", fn);
  const size_t need = oq_workspace_bytes(OQ_OP_LINEAR, M, K, N, afmt);
  if (need > NOALLOC_BYTES)
    return fail(OQ_ERR_WORKSPACE, "%s: this layer needs %zu bytes of scratch; the static scratch holds %zu (use "
                "oq_linear_fused with a workspace)", fn, need, NOALLOC_BYTES);
  void *ws = nullptr;
  int rc = scratch_for_current_device(fn, &ws);
  if (rc) return rc;
  return linear_fused_impl(fn, x, M, K, ldx, rot, center, afmt, w, w_scale, N, group, w1, bias, y, ldy, ws,
                           NOALLOC_BYTES, stream);
}

// ------------------------------------------------------------ Lloyd-Max path
int oq_lloyd_max_levels(int32_t d, int32_t bits, double *levels) {
  int rc = check_lm_bits("oq_lloyd_max_levels", bits);
  if (rc) return rc;
  if (d < 3) return fail(OQ_ERR_INVALID_ARG, "oq_lloyd_max_levels: d=%d must be >= 3", d);
  if (!levels) return fail(OQ_ERR_INVALID_ARG, "oq_lloyd_max_levels: levels is NULL");
  const double res = lloyd_max_solve(d, bits, levels);
  if (!(res >= 0.0) || res > 1e-10)
    return fail(OQ_ERR_UNSUPPORTED, "oq_lloyd_max_levels: no convergence for d=%d bits=%d (residual %g)", d, bits, res);
  g_err[0] = 0;
  return OQ_OK;
}

int oq_lloyd_max_tables(int32_t d, int32_t bits, uint16_t *levels_f16, float *thresholds) {
  if (!levels_f16 || !thresholds) return fail(OQ_ERR_INVALID_ARG, "oq_lloyd_max_tables: NULL output");
  int rc = check_lm_bits("oq_lloyd_max_tables", bits);
  if (rc) return rc;
  double lv[256];
  rc = oq_lloyd_max_levels(d, bits, lv);
  if (rc) return rc;
  const int L = 1 << bits;
  for (int i = 0; i < L; ++i) levels_f16[i] = f64_to_f16_rne(lv[i]);
  for (int i = 0; i + 1 < L; ++i) {
    const float a = f16_to_f32(levels_f16[i]), b = f16_to_f32(levels_f16[i + 1]);
    if (!(a < b)) return fail(OQ_ERR_UNSUPPORTED, "oq_lloyd_max_tables: float16 levels %d, %d coincide", i, i + 1);
    thresholds[i] = (a + b) * 0.5f;
    if ((double)thresholds[i] != 0.5 * ((double)a + (double)b))
      return fail(OQ_ERR_UNSUPPORTED, "oq_lloyd_max_tables: midpoint %d is not exact in float32", i);
  }
  g_err[0] = 0;
  return OQ_OK;
}

size_t oq_tiled_f16_bytes(int64_t rows, int32_t K) {
  if (rows < 0 || K <= 0 || K % 16) return 0;
  return (size_t)tiled_f16_bytes(rows, K);
}

int oq_quant_act_lm(const uint16_t *x, int64_t M, int32_t d, int64_t ldx, const oq_rot *rot, int center,
                    int32_t bits, int tiled, const uint16_t *levels_f16, const float *thresholds, void *codes,
                    int64_t ldc_bytes, float *scale, float *mean, hipStream_t stream) {
  const char *fn = "oq_quant_act_lm";
  int rc = check_x(fn, x, M, d, ldx);
  if (rc) return rc;
  rc = check_lm_bits(fn, bits);
  if (rc) return rc;
  if (!rpbh_wave_supported(d)) return fail(OQ_ERR_UNSUPPORTED, "%s: d=%d must be at most 4096", fn, d);
  if (M == 0) return OQ_OK;
  if (!codes || !scale) return fail(OQ_ERR_INVALID_ARG, "%s: codes or scale is NULL", fn);
  if (!levels_f16 || !thresholds) return fail(OQ_ERR_INVALID_ARG, "%s: the codebook tables are NULL", fn);
  if ((reinterpret_cast<uintptr_t>(levels_f16) & 1) || (reinterpret_cast<uintptr_t>(thresholds) & 3))
    return fail(OQ_ERR_ALIGNMENT, "%s: codebook tables misaligned", fn);
  if (!al16(codes)) return fail(OQ_ERR_ALIGNMENT, "%s: codes must be 16-byte aligned", fn);
  if (!tiled) {
    if (ldc_bytes % 16) return fail(OQ_ERR_ALIGNMENT, "%s: code rows must be 16-byte aligned", fn);
    if (ldc_bytes < (bits <= 4 ? d / 2 : d)) return fail(OQ_ERR_INVALID_ARG, "%s: ldc_bytes too small", fn);
  }
  if (center && !mean) return fail(OQ_ERR_INVALID_ARG, "%s: centering needs mean", fn);
  RotArgs ra;
  rc = rot_args(fn, rot, d, &ra);
  if (rc) return rc;
  if (ra.kron_m) return fail(OQ_ERR_UNSUPPORTED, "%s: Lloyd-Max codes with the Kronecker rotation", fn);
  const LmArgs la{bits, thresholds, levels_f16};
  const int mode = tiled ? OUT_LMF16 : (bits <= 4 ? OUT_LM4 : OUT_LM8);
  g_err[0] = 0;
  return hip_status(launch_rpbh_quant(x, M, d, ldx, ra, center ? 1 : 0, mean, mode, 0, codes, tiled ? 0 : ldc_bytes,
                                      scale, stream, nullptr, &la),
                    fn);
}

int oq_prepack_w16(const uint8_t *w, const float *w_scale, int32_t N, int32_t K, int32_t group, uint16_t *w16_tiled,
                   hipStream_t stream) {
  const char *fn = "oq_prepack_w16";
  if (N < 0) return fail(OQ_ERR_INVALID_ARG, "%s: N < 0", fn);
  if (K <= 0 || K % 32) return fail(OQ_ERR_UNSUPPORTED, "%s: K=%d must be a positive multiple of 32", fn, K);
  if (group < 32 || group % 32 || K % group)
    return fail(OQ_ERR_UNSUPPORTED, "%s: group=%d must be a multiple of 32 dividing K=%d", fn, group, K);
  if (N > 0 && (!w || !w_scale || !w16_tiled)) return fail(OQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!al16(w) || !al16(w16_tiled)) return fail(OQ_ERR_ALIGNMENT, "%s: misaligned", fn);
  g_err[0] = 0;
  return hip_status(launch_prepack_w16(w, w_scale, N, K, group, reinterpret_cast<uint8_t *>(w16_tiled), stream), fn);
}

int oq_gemm_lm(int32_t bits, int tiled, const void *qa, int64_t lda_bytes, const float *a_scale, int64_t M,
               int32_t K, const uint16_t *levels_f16, const uint16_t *w16_tiled, int32_t N, const float *mean,
               const float *w1, const float *bias, uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes,
               hipStream_t stream) {
  const char *fn = "oq_gemm_lm";
  int rc = check_lm_bits(fn, bits);
  if (rc) return rc;
  if (M < 0 || N < 0) return fail(OQ_ERR_INVALID_ARG, "%s: negative M or N", fn);
  if (K <= 0 || K % 32) return fail(OQ_ERR_UNSUPPORTED, "%s: K=%d must be a positive multiple of 32", fn, K);
  if ((mean == nullptr) != (w1 == nullptr)) return fail(OQ_ERR_INVALID_ARG, "%s: mean and w1 must be given together", fn);
  if (M == 0 || N == 0) return OQ_OK;
  if (!qa || !a_scale || !w16_tiled || !y) return fail(OQ_ERR_INVALID_ARG, "%s: NULL operand", fn);
  if (!al16(qa) || !al16(w16_tiled)) return fail(OQ_ERR_ALIGNMENT, "%s: operands must be 16-byte aligned", fn);
  if (ldy < N) return fail(OQ_ERR_INVALID_ARG, "%s: ldy=%lld < N=%d", fn, (long long)ldy, N);
  if (reinterpret_cast<uintptr_t>(y) & 1) return fail(OQ_ERR_ALIGNMENT, "%s: y misaligned", fn);
  const uint8_t *A = static_cast<const uint8_t *>(qa);
  g_err[0] = 0;
  if (!tiled) {
    if (lda_bytes % 16 || lda_bytes < (bits <= 4 ? K / 2 : K))
      return fail(OQ_ERR_INVALID_ARG, "%s: lda_bytes must be a multiple of 16 covering a row of codes", fn);
    if (!levels_f16 || (reinterpret_cast<uintptr_t>(levels_f16) & 1))
      return fail(OQ_ERR_INVALID_ARG, "%s: canonical codes need the float16 levels", fn);
    const size_t need = (size_t)tiled_f16_bytes(M, K);
    if (!ws || ws_bytes < need || !al16(ws))
      return fail(OQ_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) needed", fn, need);
    rc = hip_status(launch_lm_expand(A, lda_bytes, bits <= 4, levels_f16, 1 << bits, M, K,
                                     static_cast<uint8_t *>(ws), stream), fn);
    if (rc) return rc;
    A = static_cast<const uint8_t *>(ws);
  }
  return hip_status(launch_gemm_f16(A, a_scale, M, K, reinterpret_cast<const uint8_t *>(w16_tiled), N, mean, w1,
                                    bias, y, ldy, stream),
                    fn);
}

// ------------------------------------------------------ asymmetric weights
int oq_quant_weight_asym(const float *w, int32_t N, int32_t K, int64_t ldw, const oq_rot *rot, int32_t group,
                         uint8_t *codes, uint16_t *sigma, uint16_t *zero, float *w1, hipStream_t stream) {
  const char *fn = "oq_quant_weight_asym";
  if (N < 0) return fail(OQ_ERR_INVALID_ARG, "%s: N < 0", fn);
  if (K < 64 || K > 16384 || K % 64) return fail(OQ_ERR_UNSUPPORTED, "%s: K=%d must be a multiple of 64 in [64, 16384]", fn, K);
  if (group < 32 || group % 32 || K % group)
    return fail(OQ_ERR_UNSUPPORTED, "%s: group=%d must be a multiple of 32 dividing K=%d", fn, group, K);
  if (N == 0) return OQ_OK;
  if (!w || !codes || !sigma || !zero) return fail(OQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (ldw < K) return fail(OQ_ERR_INVALID_ARG, "%s: ldw < K", fn);
  if (!al16(w) || (ldw * 4) % 16 || !al16(codes)) return fail(OQ_ERR_ALIGNMENT, "%s: rows must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(sigma) | reinterpret_cast<uintptr_t>(zero)) & 1)
    return fail(OQ_ERR_ALIGNMENT, "%s: sigma/zero misaligned", fn);
  RotArgs ra;
  int rc = rot_args(fn, rot, K, &ra);
  if (rc) return rc;
  if (rot_out_width(ra, K) % group)
    return fail(OQ_ERR_UNSUPPORTED, "%s: group=%d must divide the rotated width %d", fn, group, rot_out_width(ra, K));
  g_err[0] = 0;
  return hip_status(launch_weight_rpbh_asym(w, N, K, ldw, ra, group, codes, sigma, zero, w1, stream), fn);
}

int oq_prepack_w4_asym(const uint8_t *w, const uint16_t *sigma, const uint16_t *zero, int32_t N, int32_t K,
                       int32_t group, uint8_t *w_tiled, float *w_scale_t, uint32_t *corr, hipStream_t stream) {
  const char *fn = "oq_prepack_w4_asym";
  if (N < 0) return fail(OQ_ERR_INVALID_ARG, "%s: N < 0", fn);
  if (K <= 0 || K % 64) return fail(OQ_ERR_UNSUPPORTED, "%s: K=%d must be a positive multiple of 64", fn, K);
  if (group != 64) return fail(OQ_ERR_UNSUPPORTED, "%s: group must be 64 (got %d)", fn, group);
  if (N > 0 && (!w || !sigma || !zero || !w_tiled || !w_scale_t || !corr))
    return fail(OQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!al16(w) || !al16(w_tiled) || (reinterpret_cast<uintptr_t>(corr) & 7))
    return fail(OQ_ERR_ALIGNMENT, "%s: misaligned", fn);
  g_err[0] = 0;
  return hip_status(launch_prepack_w4a(w, sigma, zero, N, K, w_tiled, w_scale_t, corr, stream), fn);
}

int oq_quant_act_gsum(const uint16_t *x, int64_t M, int32_t d, int64_t ldx, const oq_rot *rot, int center, int afmt,
                      void *codes, float *scale, uint32_t *gsum, float *mean, hipStream_t stream) {
  const char *fn = "oq_quant_act_gsum";
  int rc = check_x(fn, x, M, d, ldx);
  if (rc) return rc;
  PctlArgs pa;
  const PctlArgs *pp = nullptr;
  if (afmt & OQ_SCALE_PCTL) {
    afmt &= ~OQ_SCALE_PCTL;
    rc = pctl_setup(fn, afmt, d, &pa);
    if (rc) return rc;
    pp = &pa;
  }
  if (afmt != (OQ_A4 | OQ_TILED) && afmt != (OQ_A6 | OQ_TILED))
    return fail(OQ_ERR_UNSUPPORTED, "%s: group sums come with OQ_A4 | OQ_TILED or OQ_A6 | OQ_TILED codes", fn);
  if (!rpbh_wave_supported(d) || d % 64)
    return fail(OQ_ERR_UNSUPPORTED, "%s: d=%d must be a multiple of 64 up to 4096", fn, d);
  if (M == 0) return OQ_OK;
  if (!codes || !scale || !gsum) return fail(OQ_ERR_INVALID_ARG, "%s: NULL output", fn);
  if (!al16(codes) || (reinterpret_cast<uintptr_t>(gsum) & 3)) return fail(OQ_ERR_ALIGNMENT, "%s: misaligned", fn);
  if (center && !mean) return fail(OQ_ERR_INVALID_ARG, "%s: centering needs mean", fn);
  RotArgs ra;
  rc = rot_args(fn, rot, d, &ra);
  if (rc) return rc;
  if (ra.kron_m) return fail(OQ_ERR_UNSUPPORTED, "%s: group sums with the Kronecker rotation", fn);
  const int base = afmt & ~OQ_TILED;
  g_err[0] = 0;
  return hip_status(launch_rpbh_quant(x, M, d, ldx, ra, center ? 1 : 0, mean, base == OQ_A4 ? OUT_FP6 : OUT_FP6X2,
                                      qmax_of(base), codes, 0, scale, stream, pp, nullptr, gsum),
                    fn);
}

int oq_gemm_w4a4_asym(int afmt, const uint8_t *qa, const float *a_scale, const uint32_t *gsum, int64_t M, int32_t K,
                      const uint8_t *w_tiled, const float *w_scale_t, const uint32_t *corr, int32_t N, const float *mean,
                      const float *w1, const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream) {
  const char *fn = "oq_gemm_w4a4_asym";
  if (afmt != (OQ_A4 | OQ_TILED)) return fail(OQ_ERR_UNSUPPORTED, "%s: afmt must be OQ_A4 | OQ_TILED", fn);
  int rc = check_gemm_common(fn, qa, 16, M, K, w_tiled, w_scale_t, N, y, ldy, 0);
  if (rc) return rc;
  if ((mean == nullptr) != (w1 == nullptr)) return fail(OQ_ERR_INVALID_ARG, "%s: mean and w1 must be given together", fn);
  if (M == 0 || N == 0) return OQ_OK;
  if (!a_scale || !gsum || !corr) return fail(OQ_ERR_INVALID_ARG, "%s: NULL scale, gsum or corr", fn);
  if (reinterpret_cast<uintptr_t>(corr) & 7) return fail(OQ_ERR_ALIGNMENT, "%s: corr must be 8-byte aligned", fn);
  if (!fp6_offsets_fit(M, N, K)) return fail(OQ_ERR_UNSUPPORTED, "%s: a tiled operand plane exceeds 4 GiB (split M or N)", fn);
  g_err[0] = 0;
  return hip_status(launch_gemm_fp6_asym(qa, a_scale, gsum, M, K, w_tiled, w_scale_t, corr, N, mean, w1, bias, y, ldy,
                                         stream),
                    fn);
}

// ------------------------------------------------------ measurement helper
size_t oq_probe_sink_elems(void) { return (size_t)probe_blocks() * 256; }

int oq_probe_mfma(int kind, int32_t iters, float *sink, double *ops, hipStream_t stream) {
  const char *fn = "oq_probe_mfma";
  if (kind < OQ_PROBE_FP6 || kind > OQ_PROBE_FP6_UPDATE) return fail(OQ_ERR_INVALID_ARG, "%s: unknown kind %d", fn, kind);
  if (iters < 1 || iters > (1 << 20)) return fail(OQ_ERR_INVALID_ARG, "%s: iters=%d must lie in [1, 2^20]", fn, iters);
  if (!sink || !ops) return fail(OQ_ERR_INVALID_ARG, "%s: NULL sink or ops", fn);
  g_err[0] = 0;
  return hip_status(launch_mfma_probe(kind, iters, sink, stream, ops), fn);
}

// ---------------------------------------------------------- Kronecker rotation
int oq_kron_plan(int32_t n, int32_t *m, int32_t *block, int32_t *n_pad) {
  if (n < 1 || n > 16384) return fail(OQ_ERR_UNSUPPORTED, "oq_kron_plan: n=%d must lie in [1, 16384]", n);
  if (!m || !block || !n_pad) return fail(OQ_ERR_INVALID_ARG, "oq_kron_plan: NULL output");
  const int orders[4] = {1, 12, 36, 44};
  int best = 0, bm = 0, bb = 0;
  for (int i = 0; i < 4; ++i) {
    int b = 16;  // blocks of at least 16 coordinates (one thread's share)
    while (orders[i] * b < n) b *= 2;
    if (best == 0 || orders[i] * b < best) {
      best = orders[i] * b;
      bm = orders[i];
      bb = b;
    }
  }
  if (best > 16384) return fail(OQ_ERR_UNSUPPORTED, "oq_kron_plan: no admissible width up to 16384 for n=%d", n);
  *m = bm;
  *block = bb;
  *n_pad = best;
  g_err[0] = 0;
  return OQ_OK;
}

}  // extern "C"



