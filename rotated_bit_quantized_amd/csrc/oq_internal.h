// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdlib>

#include "../../include/oq.h"

namespace oq {

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device (the attribute is held per device); `done` is that kernel's own
// set of flags.
inline hipError_t lds_limit_once(const void *kern, int bytes, std::atomic<bool> (&done)[64]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!done[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    done[dev].store(true, std::memory_order_release);
  }
  return hipSuccess;
}

// ------------------------------------------------------------------ errors --
void set_error(const char *fmt, ...);
int fail(int code, const char *fmt, ...);

// ------------------------------------------------------- numeric helpers --
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// float32 -> bfloat16 bits, IEEE round to nearest even (gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Row c' of the Paley factor H_m of the Kronecker rotation as a sign mask
// (bit c set where H_m[c'][c] = -1), from the textbook constructions with
// chi the quadratic character mod q (Euler's criterion) and the Jacobsthal
// entries Q[i][j] = chi(j - i): m = 12, 44: type I, q = 11, 43,
// H = I + [[0, 1^T], [-1, Q]]; m = 36: type II, q = 17, C = [[0, 1^T], [1, Q]],
// H = [[C + I, C - I], [C - I, -C - I]] (CentriQ Sec. 3 "Hadamard rotation",
// App. B.1).  m = 1 gives 0.
__host__ __device__ constexpr int qchar(int a, int q) {
  a %= q;
  if (a < 0) a += q;
  if (a == 0) return 0;
  int r = 1, b = a, e = (q - 1) / 2;
  while (e) {
    if (e & 1) r = (r * b) % q;
    b = (b * b) % q;
    e >>= 1;
  }
  return r == 1 ? 1 : -1;
}

__host__ __device__ constexpr uint64_t paley_row_mask(int m, int cp) {
  if (m == 1) return 0;
  uint64_t msk = 0;
  if (m == 12 || m == 44) {
    const int q = m - 1;
    for (int c = 0; c < m; ++c) {
      int v = 0;
      if (cp == 0) v = 1;
      else if (c == 0) v = -1;
      else if (c == cp) v = 1;
      else v = qchar(c - cp, q);
      if (v < 0) msk |= (uint64_t)1 << c;
    }
  } else {  // m == 36, q = 17
    const int bi = cp / 18, i = cp % 18;
    for (int c = 0; c < m; ++c) {
      const int bj = c / 18, j = c % 18;
      const int cij = (i == 0 && j == 0) ? 0 : (i == 0 || j == 0) ? 1 : (i == j ? 0 : qchar(j - i, 17));
      const int dij = i == j ? 1 : 0;
      const int v = (bi == 0 && bj == 0) ? cij + dij : (bi == 1 && bj == 1) ? -cij - dij : cij - dij;
      if (v < 0) msk |= (uint64_t)1 << c;
    }
  }
  return msk;
}

// FP6 E2M3 bit pattern of an integer code q in [-7, 7] (exact: sign bit 5,
// exponent bits 4..3 with bias 1, mantissa bits 2..0).  The magnitude goes
// through an 8-entry byte table held in two dwords (v_perm_b32).
// Global -> LDS copies: each lane moves 16 (or 4) bytes from its own global
// address to lds_addr + lane * 16 (or * 4); lds_addr is wave-uniform and goes
// to M0.  Written as inline asm on purpose: the compiler would otherwise
// treat the copy as an LDS store of unknown extent and wait for every copy in
// flight before each later LDS read, which turns a multi-stage ring into a
// serial one.  Callers order copies and reads with explicit vmcnt waits and
// workgroup barriers.  The asm has no register outputs.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_lds16(const void *g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4(const void *g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// byte address of an LDS object, for dma_lds*
__device__ __forceinline__ uint32_t lds_addr_of(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

__device__ __forceinline__ uint32_t fp6_e2m3_of_int(int q) {
  const uint32_t a = (uint32_t)(q < 0 ? -q : q);
  // |q| = 0..7 -> 0x00 0x08 0x10 0x14 0x18 0x1A 0x1C 0x1E
  const uint32_t code = __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, a) & 0xFFu;
  return code | (q < 0 ? 0x20u : 0u);
}

// bytes of one plane of the tiled FP6 operand layout (rows padded to 32)
__host__ __device__ inline int64_t tiled_bytes(int64_t rows, int K) { return (rows + 31) / 32 * (K / 64) * 1536; }
// The tiled FP6 GEMM addresses each operand with 32-bit offsets from its base:
// one plane of activations and the weights must each stay below 4 GiB.
inline bool fp6_offsets_fit(int64_t M, int N, int K) {
  return tiled_bytes(M, K) < (int64_t(1) << 32) && tiled_bytes(N, K) < (int64_t(1) << 32);
}

// activation code formats used inside the library (values of the public enum
// for the integer widths; internal operand layouts are separate constants)
enum OutMode : int {
  OUT_F32 = 0,   // float32 rotated values (oq_rotate / oq_center)
  OUT_I8 = 1,    // int8 codes (A8, A6)
  OUT_I4 = 2,    // packed nibbles (A4)
  OUT_W4G = 3,   // per-group INT4 codes + scales (offline weight fold)
  OUT_FP6 = 4,   // A4 codes as FP6 E2M3 in the tiled MFMA operand layout
  OUT_FP6X2 = 5, // A6 codes split q = 8 qh + ql into two tiled FP6 planes
  OUT_LM4 = 6,   // Lloyd-Max level indices, packed two per byte (bits <= 4)
  OUT_LM8 = 7,   // Lloyd-Max level indices, one byte each (bits <= 8)
  OUT_LMF16 = 8, // Lloyd-Max levels as float16 in the tiled f16 MFMA layout
  OUT_W4A = 9,   // asymmetric INT4 per group: codes Q - 8, bfloat16 scale and shift (weights)
};

// bytes of the tiled float16 operand layout: rows padded to 32, one 1 KiB
// chunk per (32 rows, 16 k); lane l of a chunk holds row l % 32, k 8 (l / 32)
// .. + 7 as 8 consecutive float16
__host__ __device__ inline int64_t tiled_f16_bytes(int64_t rows, int K) { return (rows + 31) / 32 * 32 * (int64_t)K * 2; }

// -------------------------------------------------------- kernel launchers --
struct RotArgs {
  int rounds;            // 0 = no rotation
  int block;             // h
  const int32_t *perm;   // [rounds][d]
  const int8_t *signs;   // [rounds][d]
  float c_h;             // RN32(1/sqrt h); for the Kronecker rotation RN32(1/sqrt(m h))
  int kron_m = 0;        // 0: RPBH rounds; else the order m of the Paley factor of (H_m (x) H_h)
};

// width of the rotated (and quantized) row: the padded m h for the Kronecker rotation
inline int rot_out_width(const RotArgs &ra, int d) { return ra.kron_m ? ra.kron_m * ra.block : d; }

// Percentile range of a token (CentriQ Sec. 4.2 "Scale and grid"):
// r = RN32((q * gamma) / z), q = lo + frac (hi - lo) in float64, where lo and
// hi are the rank-th and (rank-1)-th largest magnitudes of the row.
struct PctlArgs {
  int rank;     // 2..4 for rows of at most 4096
  double frac;  // rho (n - 1) - floor(rho (n - 1))
  double gamma;
  double z;     // Phi^-1((1 + rho) / 2)
};

// Lloyd-Max codes (OrbitQuant's activation codebook): the token's RMS scale
// and the nearest of 2^bits stored float16 levels, decided by the float32
// thresholds between them (ascending, device memory).
struct LmArgs {
  int bits;                // 1..8
  const float *thr;        // [2^bits - 1]
  const uint16_t *levels;  // [2^bits] float16 bits
};

// K1: (center) -> RPBH rounds -> (quantize) per token row; pctl selects the
// percentile range instead of absmax (integer outputs, rows the wave kernel
// takes only); the OUT_LM* modes take their codebook from lm (wave kernel
// only); gsum (tiled FP6 modes, wave kernel only), if set, receives the sum p
// of the codes of every 64-wide group, group-major [d/64][M], as one word of
// two bfloat16 pieces (8 floor(p / 8) in bits 0-15, the rest in bits 16-31).
hipError_t launch_rpbh_quant(const uint16_t *x, int64_t M, int d, int64_t ldx,
                             const RotArgs &rot, int center, float *mean,
                             int out_mode, int qmax, void *out, int64_t ld_out_bytes,
                             float *scale, hipStream_t stream, const PctlArgs *pctl = nullptr,
                             const LmArgs *lm = nullptr, uint32_t *gsum = nullptr);

// K1, one wavefront per row (activation rows of width d <= 4096).
bool rpbh_wave_supported(int d);
// Factorised rotation on the wave kernel: Paley order km and Sylvester
// block b with km = 1, b <= 1024 or b in {2048, 4096}; km = 12, b in {64,
// 128, 256}; or km in {36, 44}, b = 64; and a native width din that is a
// multiple of 16.
bool rpbh_wave_kron_supported(int km, int b, int din);
hipError_t launch_rpbh_wave_kron(const uint16_t *x, int64_t M, int din, int64_t ldx, const RotArgs &rot, int center,
                                 float *mean, int mode, int qmax, void *out, int64_t ld_out_bytes, float *scale,
                                 hipStream_t stream);
hipError_t launch_rpbh_wave(const uint16_t *x, int64_t M, int d, int64_t ldx, const RotArgs &rot, int center,
                            float *mean, int mode, int qmax, void *out, int64_t ld_out_bytes, float *scale,
                            hipStream_t stream, const PctlArgs *pctl = nullptr, const LmArgs *lm = nullptr,
                            uint32_t *gsum = nullptr);

// K2: dense per-32 transform -> (MXFP4 quantize | float32 out); mx_out: 0 float32,
// 1 row-major codes + E8M0, 2 tiled MXFP4 layout.
hipError_t launch_dense32(const uint16_t *x, int64_t M, int d, int64_t ldx,
                          const uint16_t *mats, int mx_out, void *out, int64_t ld_out_bytes,
                          uint8_t *e8m0, hipStream_t stream);

// K3/K4: integer-coded activations x packed INT4 weights, fp32 group epilogue.
//   a_is_nibble: activations packed two per byte (A4) instead of int8.
//   ws: for int8 activations, scratch of float32 partial sums; with at least
//   int_gemm_splits(M, N, K, group) x M x N x 4 bytes a small product runs
//   split across K (then the partial sums are added in split order);
//   otherwise, or when NULL, in one pass.
hipError_t launch_gemm_int(const void *qa, int64_t lda_bytes, int a_is_nibble,
                           const float *a_scale, int64_t M, int K,
                           const uint8_t *w, const float *w_scale, int N, int group,
                           const float *mean, const float *w1, const float *bias,
                           uint16_t *y, int64_t ldy, hipStream_t stream, void *ws = nullptr,
                           size_t ws_bytes = 0);
// Workgroups of the W4A8 GEMM across K: enough 128 x 128 tiles fill the
// device alone; below half of its 256 CUs, the groups are split so that
// every CU gets a workgroup (at most one split per group).
inline int int_gemm_splits(int64_t M, int N, int K, int group) {
  if (M <= 0 || N <= 0 || K <= 0 || group <= 0) return 1;
  const int64_t tiles = ((N + 127) / 128) * ((M + 127) / 128);
  if (tiles >= 128) return 1;
  int64_t s = (256 + tiles - 1) / tiles;
  if (s > K / group) s = K / group;
  return s < 1 ? 1 : (int)s;
}
// Small W4A8 products (8-bit activations, fewer 128 x 128 tiles than half the
// CUs, K <= 4096) run one 4-wave workgroup per 32 x 32 output tile over the
// whole of K, with no scratch.  OQ_INT_SMALL=0 in the environment turns this
// off (then the split or one-pass kernel runs them).
inline bool int_gemm_small(int64_t M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0 || K > 4096) return false;
  if (((N + 127) / 128) * ((M + 127) / 128) >= 128) return false;
  const char *e = getenv("OQ_INT_SMALL");
  return !(e && e[0] == '0');
}
// scratch that lets every group size split (0 when the product needs none)
inline size_t int_gemm_split_bytes(int64_t M, int N, int K) {
  if (int_gemm_small(M, N, K)) return 0;
  const int s = int_gemm_splits(M, N, K, 32);  // the most splits any group allows
  return s > 1 ? (size_t)s * (size_t)M * (size_t)N * 4 : 0;
}

// Tiled FP6 GEMM (A4: planes = 1, A6: planes = 2); weights from prepack.
hipError_t launch_gemm_fp6(const uint8_t *A, int planes, const float *a_scale, int64_t M, int K, const uint8_t *W,
                           const float *wst, int N, const float *mean, const float *w1, const float *bias,
                           uint16_t *y, int64_t ldy, hipStream_t stream);
hipError_t launch_prepack_w4(const uint8_t *w, const float *ws, int N, int K, uint8_t *out, float *out_s,
                             hipStream_t stream);
// Tiled A4 x asymmetric INT4 weights (codes q'/2 with weight scale 2^1), with
// F initialised to -sum_g corr[o][g] gsum[t][g] (single plane, group 64)
hipError_t launch_gemm_fp6_asym(const uint8_t *A, const float *a_scale, const uint32_t *gsum, int64_t M, int K,
                                const uint8_t *W, const float *wst, const uint32_t *corr, int N, const float *mean,
                                const float *w1, const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream);
// canonical asymmetric codes + bfloat16 sigma, z -> tiled q'/2, sigma [G][Np],
// -C as three bfloat16 pieces [G][Np][2] (uint32 pairs)
hipError_t launch_prepack_w4a(const uint8_t *w, const uint16_t *sig, const uint16_t *zero, int N, int K, uint8_t *out,
                              float *out_s, uint32_t *out_c, hipStream_t stream);

// K5: MXFP4 x MXFP4 with E8M0 block scales (scaled FP4 MFMA); tiled_in: both
// operands in the tiled MXFP4 layout (codes + scale words), else row-major.
hipError_t launch_gemm_mx(int tiled_in, const uint8_t *qa, int64_t lda_bytes, const uint8_t *a_e8m0,
                          int64_t M, int K, const uint8_t *w, const uint8_t *w_e8m0, int N,
                          const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream);
hipError_t launch_prepack_mx(const uint8_t *w, const uint8_t *w_e8m0, int N, int K, uint8_t *out, uint8_t *out_s,
                             hipStream_t stream);
// bytes of the tiled MXFP4 codes of `rows` rows (rows padded to 32); the
// scale words take a sixteenth of that
inline int64_t tiled_mx_bytes(int64_t rows, int K) { return (rows + 31) / 32 * 32 * (int64_t)(K / 2); }

// Lloyd-Max activation GEMM: tiled float16 levels x tiled W16 (float16 MFMA,
// float32 sums), epilogue rho F + m w1 + b; K a multiple of 32.
hipError_t launch_gemm_f16(const uint8_t *A, const float *a_scale, int64_t M, int K, const uint8_t *W, int N,
                           const float *mean, const float *w1, const float *bias, uint16_t *y, int64_t ldy,
                           hipStream_t stream);
// canonical INT4 weights + group scales -> tiled W16 = RN16(s q)
hipError_t launch_prepack_w16(const uint8_t *w, const float *ws, int N, int K, int group, uint8_t *out,
                              hipStream_t stream);
// canonical Lloyd-Max codes -> tiled float16 levels
hipError_t launch_lm_expand(const uint8_t *codes, int64_t ldc, int nibbles, const uint16_t *levels, int nlev,
                            int64_t M, int K, uint8_t *out, hipStream_t stream);

// Host: Lloyd-Max levels of the unit-variance sphere marginal of width d
// (ascending, 2^bits), solved to the fixed point of Lloyd's conditions;
// returns the final max residual, or a negative value on failure.
double lloyd_max_solve(int d, int bits, double *levels);

// Offline weight preparation.
hipError_t launch_weight_rpbh(const float *w, int N, int K, int64_t ldw, const RotArgs &rot,
                              int group, uint8_t *codes, float *scales, float *w1,
                              hipStream_t stream);
// asymmetric INT4 per group (CentriQ Eq. 2, RTN min-max): codes Q - 8 packed
// [N][K/2], bfloat16 scale and shift [N][K/group] each
hipError_t launch_weight_rpbh_asym(const float *w, int N, int K, int64_t ldw, const RotArgs &rot, int group,
                                   uint8_t *codes, uint16_t *sigma, uint16_t *zero, float *w1, hipStream_t stream);
hipError_t launch_weight_dense32(const float *w, int N, int K, int64_t ldw, const uint16_t *mats,
                                 uint8_t *codes, uint8_t *e8m0, float *w1, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cus();
// Matrix-core rate probe (oq_probe_mfma): launches it and returns the number
// of operations (2 M N K per instruction) one launch performs in *ops.
hipError_t launch_mfma_probe(int kind, int iters, float *sink, hipStream_t stream, double *ops);
int probe_blocks();

}  // namespace oq
