/*
 * oq.h -- C ABI of the rotated low-bit linear layer for AMD MI355X (gfx950).
 *
 * The layer (CentriQ, arXiv 2610.06260, Sec. 4.2 Eq. 5 and App. B.2 Eq. 9;
 * OrbitQuant PR #25, "Default changes" and "Runtime work"):
 *
 *     y_t = alpha_t * sum_g s_w[o,g] * (q_a . q_w)_g  +  m_t * w1[o]  +  b[o]
 *     q_a = Q_a( R (x_t - m_t 1) )
 *
 * R is a randomised permuted block-Hadamard rotation (one or two rounds of
 * gather -> +-1 signs -> normalised Sylvester blocks of h = 32..1024) or a set
 * of dense per-32-block transforms (WUSH review, "Core claim"); Q_a is the
 * per-token absmax quantizer of CentriQ Eq. 1 (8, 6 or 4 bits) or MXFP4
 * (E2M1 elements, one E8M0 scale per 32); weights are symmetric INT4 with
 * one fp32 scale per row and group of input columns, or MXFP4.
 *
 * Conventions shared by every call
 *   - Return value: OQ_OK (0) or one of the OQ_ERR_* codes.  On error nothing
 *     has been enqueued; oq_last_error() returns a message for the calling
 *     thread.  There is no fallback path: an unsupported request fails
 *     (model card FLUX.1-schnell-OrbitQuant-W4A4, "Limitations": the fused
 *     runtime fails loudly when its kernel is unavailable).
 *   - Every data pointer is device memory owned by the caller.  The library
 *     allocates no device memory except where a call says so
 *     (oq_linear_fused with ws == NULL is rejected, not allocated).
 *     Descriptor structs (oq_rot) are host memory, read during the call only.
 *   - Calls are asynchronous on the caller's stream; none synchronises.
 *   - Matrices are row-major.  Leading dimensions are in elements unless the
 *     name ends in _bytes.  bfloat16 values are passed as uint16_t bits.
 *   - Alignment: x, y and code/weight pointers 16 bytes; leading dimensions
 *     such that every row starts 16-byte aligned.  Violations give
 *     OQ_ERR_ALIGNMENT.
 *   - Thread safety: calls may be made from several host threads; calls on
 *     one stream execute in order.
 */
#ifndef OQ_H
#define OQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  OQ_OK = 0,
  OQ_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad enum value       */
  OQ_ERR_UNSUPPORTED = 2,   /* well-formed request this library does not run */
  OQ_ERR_ALIGNMENT = 3,     /* pointer or leading dimension misaligned      */
  OQ_ERR_WORKSPACE = 4,     /* workspace missing or too small               */
  OQ_ERR_HIP = 5            /* the HIP runtime reported a launch error      */
};

/* rotation kinds */
enum { OQ_ROT_RPBH = 1, OQ_ROT_DENSE32 = 2, OQ_ROT_KRON = 3 };

/* activation code formats (the value is the bit width for integer codes) */
enum { OQ_A8 = 8, OQ_A6 = 6, OQ_A4 = 4, OQ_MXFP4 = 0x104 };

/* weight formats for oq_quant_weight */
enum { OQ_W4 = 4, OQ_W_MXFP4 = 0x104 };

/*
 * Operand layout flag, OR-ed into afmt (OQ_A4 | OQ_TILED, OQ_A6 | OQ_TILED):
 * codes are stored as FP6 E2M3 values of the integer codes (exact for
 * |q| <= 7) in the MFMA-tiled layout below, the layout the fast GEMM reads.
 *   rows padded to a multiple of 32, K a multiple of 64; tile (r/32, kg =
 *   k / 64) is 1536 bytes at ((r/32) * (K/64) + kg) * 1536.  Within it, the
 *   32 codes of row r and k-half h (k = 64 kg + 32 h + j, j = 0..31) form a
 *   192-bit string with code j in bits [6j, 6j+6); with l = 32 h + r % 32,
 *   its bytes 0..15 sit at tile + 16 l and bytes 16..23 at tile + 1024 + 8 l.
 *   One plane is oq_tiled_bytes(rows, K) bytes.  OQ_A6 uses two planes:
 *   q = 8 qh + ql with qh = floor(q / 8) in plane 0 and ql = q - 8 qh in
 *   plane 1 (each in [-4, 7]).
 * Weights for tiled GEMMs come from oq_prepack_w4 (same layout, one plane,
 * plus scales transposed to [K/64][N_padded]).  The per-token scale
 * (a_scale) and mean arrays are unchanged.  Tiled GEMMs require group == 64.
 *
 * OQ_MXFP4 | OQ_TILED (K a multiple of 128): the MXFP4 codes and E8M0 scales
 * in the layout the MXFP4 GEMM copies whole:
 *   codes: rows padded to 32; tile (r/32, kg = k / 64) is 1024 bytes at
 *     ((r/32) * (K/64) + kg) * 1024; the 16 bytes of row r and k-half h (32
 *     E2M1 codes, code j in bits [4j, 4j+4), the bytes of the row-major
 *     layout) sit at tile + 16 (32 h + r % 32).  oq_tiled_mx_bytes(rows, K).
 *   scales: one 32-bit word per (128-wide k-slice s, row r) at byte
 *     (s * rows_padded + r) * 4, holding the E8M0 bytes of the blocks
 *     4s .. 4s+3 in order; oq_tiled_mx_bytes(rows, K) / 16 bytes, 4-byte
 *     aligned.  Padding rows carry zero codes.
 * Weights come from oq_prepack_mx.
 */
enum { OQ_TILED = 0x10000 };

/*
 * Scale flag, OR-ed into afmt for integer activation codes (OQ_A8, OQ_A6,
 * OQ_A4, tiled or not) in oq_quant_act and oq_linear_fused -- CentriQ Sec.
 * 4.2 "Scale and grid" and App. B.3 Table 3: the token's range is
 *   r = RN32((q * 2.5591) / Phi^-1(0.99975))      (evaluated in float64),
 * q the 0.9995-quantile of the d rotated magnitudes, interpolated linearly
 * between the order statistics floor(0.9995 (d - 1)) and the next one
 * (ascending); then alpha = RN32(r / qmax) and codes clip to +-qmax as in
 * Eq. 1.  Needs d % 16 == 0 and 16 <= d <= 4096; not for MXFP4.
 */
enum { OQ_SCALE_PCTL = 0x20000 };

/* Bytes of one plane of the tiled FP6 layout for `rows` rows of width K. */
size_t oq_tiled_bytes(int64_t rows, int32_t K);

/* Bytes of the tiled MXFP4 codes for `rows` rows of width K (the scale words
 * take a sixteenth of that). */
size_t oq_tiled_mx_bytes(int64_t rows, int32_t K);

/*
 * Rotation descriptor (host struct, device arrays).
 *
 * OQ_ROT_RPBH -- OrbitQuant PR #25 "Default changes" (independent extra
 *   rounds); CentriQ related-work paragraph (randomly permuted block-Hadamard
 *   basis); model card "Artifact Files" (stored deterministic rotation
 *   metadata).  Round r maps v to B_h D_{s_r} P_{pi_r} v:
 *     u[i] = signs[r][i] * v[perm[r][i]]    (gather over the whole width d)
 *     v    = (1/sqrt h) H_h u  per block of h consecutive coordinates.
 *   block: power of two in [32, 1024]; d % block == 0; rounds in {1, 2};
 *   perm: int32 [rounds][d], each row a permutation of 0..d-1 (not checked);
 *   signs: int8 [rounds][d] in {-1, +1}.
 *   The float32 results follow one fixed order: butterfly stages of stride
 *   1, 2, ..., h/2, each add/subtract rounded once, then a multiply by
 *   RN32(1/sqrt h).
 *
 * OQ_ROT_DENSE32 -- WUSH review "Core claim": one transform per 32-block,
 *   activations take T_b and weights its inverse-transpose T_b^{-T}.
 *   mats: bfloat16 [d/32][32][32] row-major, v_b = T_b x_b, 16-byte aligned.
 *   d % 32 == 0.  Weights (oq_quant_weight) use the same mats: the library
 *   forms T_b^{-T} itself in float64 (Gauss-Jordan with partial pivoting);
 *   every T_b must be invertible.
 *   Activation-side float32 results are T_b x_b rounded once to float32,
 *   the bf16 x bf16 products summed in float64 (exact whenever the products
 *   of one output span at most 32 binades, as ordinary activations do).
 */
typedef struct {
  int32_t kind;
  int32_t d;
  int32_t block;
  int32_t rounds;
  const int32_t *perm;
  const int8_t *signs;
  const uint16_t *mats;
} oq_rot;

/* Message of the last failed call on this thread ("" if none). */
const char *oq_last_error(void);

/*
 * oq_center -- CentriQ Sec. 4.2 Eq. 4: per-token mean and centered token.
 *   mean[t] = RN32(RN64(sum_j x[t][j]) / d), the sum formed in float64
 *             (exact whenever the row's exponent spread allows, which holds
 *             for ordinary activations);
 *   xc[t][j] = RN32(x[t][j] - mean[t]).
 * x: bf16 [M][ldx]; xc: float32 [M][ldxc] (may be NULL to compute the mean
 * only); mean: float32 [M].  M >= 0 (M == 0 enqueues nothing); 1 <= d <= 16384.
 */
int oq_center(const uint16_t *x, int64_t M, int32_t d, int64_t ldx,
              float *xc, int64_t ldxc, float *mean, hipStream_t stream);

/*
 * oq_rotate -- the rotation of the online activation path (OrbitQuant PR #25
 * "Runtime work": the whole pre-rotation in one kernel) with float32 output,
 * optionally after centering (CentriQ Eq. 4-5: rotate the centered token).
 * rot: required (RPBH or DENSE32); rot->d is the width.
 * x: bf16 [M][ldx]; y: float32 [M][ldy]; mean: float32 [M], required iff
 * center != 0 (DENSE32 does not support centering).
 */
int oq_rotate(const oq_rot *rot, const uint16_t *x, int64_t M, int64_t ldx,
              int center, float *mean, float *y, int64_t ldy, hipStream_t stream);

/*
 * oq_quant_act -- fused (center) -> rotate -> quantize -> pack for the
 * activations: CentriQ Eq. 1 (symmetric per-token absmax, alpha_t = r_t/qmax,
 * qmax = 2^{b-1}-1) and OrbitQuant's absmax A8; MXFP4 per WUSH review.
 *   codes for q = clamp(RNE(RN32(v * RN32(qmax / a))), -qmax, qmax) with
 *   a = max(max_j |v_tj|, RN32(1e-10)) (model card: activation normalization
 *   epsilon 1e-10); scale[t] = RN32(a / qmax).
 * afmt OQ_A8, OQ_A6: int8 codes [M][ldc_bytes]; OQ_A4: two codes per byte,
 *   element 2i in bits 3..0, two's complement, [M][ldc_bytes >= d/2];
 *   scale float32 [M]; e8m0 must be NULL.
 * afmt OQ_A4 | OQ_TILED, OQ_A6 | OQ_TILED: codes in the tiled FP6 layout
 *   (planes * oq_tiled_bytes(M, d) bytes; d % 64 == 0; ldc_bytes ignored).
 * afmt OQ_MXFP4 (rot->kind must be OQ_ROT_DENSE32, center == 0): E2M1 codes
 *   two per byte as above, sign in bit 3; e8m0 uint8 [M][d/32] with
 *   e = clamp(floor(log2 amax) - 2, -127, 127), byte = e + 127; scale NULL.
 * rot may be NULL (no rotation; integer formats only, d = ldx's row width
 *   given by the d argument).  mean: float32 [M], required iff center != 0.
 */
int oq_quant_act(const uint16_t *x, int64_t M, int32_t d, int64_t ldx,
                 const oq_rot *rot, int center, int afmt,
                 void *codes, int64_t ldc_bytes, float *scale, uint8_t *e8m0,
                 float *mean, hipStream_t stream);

/*
 * oq_quant_weight -- offline weight path (CentriQ Sec. 3 "Hadamard
 * rotation": W x = (W H^T)(H x); App. B.1: the weight absorbs P^T H^T;
 * Eq. 4: w1 = W 1 in float32 from the unquantized weight).
 *   Each row w of W [N][ldw] (float32) becomes R w (the same rotation as the
 *   activations; for DENSE32 the inverse-transposes of rot->mats, applied in
 *   float64 with one rounding to float32), then:
 *   wfmt OQ_W4: symmetric absmax INT4 per (row, group of `group` input
 *     columns), codes packed two per byte [N][K/2], scales float32 [N][K/group];
 *   wfmt OQ_W_MXFP4: E2M1 codes [N][K/2] and E8M0 bytes [N][K/32] (group 32).
 *   w1 (nullable): float32 [N], RN32 of the row sum of the input W (float64
 *   accumulation).  rot may be NULL (no rotation).
 * group: multiple of 32 dividing K (OQ_W4); K % 32 == 0.
 */
int oq_quant_weight(const float *w, int32_t N, int32_t K, int64_t ldw,
                    const oq_rot *rot, int wfmt, int32_t group,
                    uint8_t *codes, void *scales, float *w1, hipStream_t stream);

/*
 * oq_gemm_w4a8 -- int8-coded activations (OQ_A8 or OQ_A6 codes) times packed
 * INT4 weights with the fp32 epilogue of CentriQ Eq. 5 / Eq. 9:
 *   y[t][o] = bf16_RNE( a_scale[t] * sum_g w_scale[o][g] * acc_g[t][o]
 *                       + mean[t] * w1[o] + bias[o] )
 *   acc_g = exact int32 sum over the group's input columns.
 * qa int8 [M][lda]; a_scale float32 [M]; w uint8 [N][K/2] (canonical
 * nibbles); w_scale float32 [N][K/group]; mean and w1 both NULL or both set;
 * bias nullable; y bf16 [M][ldy].  group: multiple of 32 dividing K.
 * A product of fewer than 128 output tiles of 128 x 128 with K <= 4096 runs
 * one 4-wavefront workgroup per 32 x 32 output tile (operands staged through
 * LDS from coalesced loads), with no scratch and the one-pass kernel's
 * arithmetic: the two give identical bits.  OQ_INT_SMALL=0 in the
 * environment turns this routing off.
 * ws/ws_bytes: optional device scratch (16-byte aligned, else
 * OQ_ERR_ALIGNMENT).  Another product of fewer than 128 such tiles (K >
 * 4096, or the routing above turned off) given at least
 * oq_workspace_bytes(OQ_OP_GEMM_W4A8, M, K, N, 0) bytes runs split across K
 * on more workgroups: each writes the float32 sum of its groups' s_g acc_g
 * to ws, and a second launch adds those sums in split order and applies the
 * epilogue (a different float32 summation order from the one-pass kernel,
 * within the same rounding bound).  Without scratch, or with less, the
 * product runs in one pass; the result is deterministic either way.
 */
int oq_gemm_w4a8(const int8_t *qa, int64_t lda, const float *a_scale, int64_t M, int32_t K,
                 const uint8_t *w, const float *w_scale, int32_t N, int32_t group,
                 const float *mean, const float *w1, const float *bias,
                 uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * oq_gemm_w4a4 -- 4-bit activations times 4-bit weights.
 *   afmt OQ_A4: qa nibbles [M][lda_bytes], a_scale float32 [M]; w canonical
 *     INT4 nibbles [N][K/2], w_scale float32 [N][K/group]; epilogue as
 *     oq_gemm_w4a8.
 *   afmt OQ_A4 | OQ_TILED or OQ_A6 | OQ_TILED: qa in the tiled layout (from
 *     oq_quant_act with the same afmt; lda_bytes ignored), w and w_scale
 *     from oq_prepack_w4, group 64; output bit-identical to the canonical
 *     path on the same codes.  The library picks the workgroup shape from
 *     M, N and the CU count; the environment variable OQ_FP6_TILE forces
 *     one, for tuning: 256x256, 256x192, 256x128w8 (eight waves), 256x128
 *     (four waves) or 128x192 for OQ_A4; 256x192 or 256x128w8 for OQ_A6.
 *     The result does not depend on the shape.  One activation plane
 *     (oq_tiled_bytes(M, K)) and the weights (oq_tiled_bytes(N, K)) must each
 *     stay below 4 GiB (the kernel's 32-bit operand offsets); larger requests
 *     fail with OQ_ERR_UNSUPPORTED (split M or N).
 *   afmt OQ_MXFP4: qa E2M1 nibbles, a_scale uint8 E8M0 [M][K/32]; w E2M1
 *     nibbles [N][K/2], w_scale uint8 E8M0 [N][K/32]; group must be 32;
 *     y = bf16_RNE( sum_blocks 2^(ea+ew) sum_k fp4(a) fp4(w) + bias[o] );
 *     mean/w1 must be NULL.
 */
int oq_gemm_w4a4(int afmt, const uint8_t *qa, int64_t lda_bytes, const void *a_scale,
                 int64_t M, int32_t K, const uint8_t *w, const void *w_scale,
                 int32_t N, int32_t group, const float *mean, const float *w1,
                 const float *bias, uint16_t *y, int64_t ldy,
                 void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * oq_linear_fused -- the whole layer: oq_quant_act into the workspace, then
 * the matching GEMM, on one stream (CentriQ App. B.2: prologue quantizes
 * each token tile once; rank-1 term and bias in the GEMM epilogue).
 * afmt OQ_A8/OQ_A6/OQ_A4 with an RPBH rotation (or NULL), optional centering
 * (then w1 is required); OQ_MXFP4 with a DENSE32 rotation and E8M0 w_scale.
 * afmt OQ_A4 | OQ_TILED or OQ_A6 | OQ_TILED: w/w_scale from oq_prepack_w4
 * (group 64); activations are quantized straight into the tiled layout.
 * ws: device scratch of at least oq_workspace_bytes(OQ_OP_LINEAR, M, K, N, afmt).
 */
int oq_linear_fused(const uint16_t *x, int64_t M, int32_t K, int64_t ldx,
                    const oq_rot *rot, int center, int afmt,
                    const uint8_t *w, const void *w_scale, int32_t N, int32_t group,
                    const float *w1, const float *bias, uint16_t *y, int64_t ldy,
                    void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * oq_linear_fused_noalloc -- oq_linear_fused for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, formats
 * and result as oq_linear_fused (bit for bit), without ws / ws_bytes: the
 * codes, scales and means go to a static scratch array of
 * OQ_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it
 * runs on until the process ends (its device address is looked up once per
 * device, on the first call there).  A layer whose
 * oq_workspace_bytes(OQ_OP_LINEAR, M, K, N, afmt) exceeds that size fails
 * with OQ_ERR_WORKSPACE before anything is enqueued.  The call allocates
 * nothing.  Every call on one GPU shares that GPU's scratch, which keeps the
 * last call's contents (nothing in it needs to start at zero): calls that
 * overlap on one GPU (several streams or host threads at once) race; serialise
 * them, for instance on one stream.
 */
#define OQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int oq_linear_fused_noalloc(const uint16_t *x, int64_t M, int32_t K, int64_t ldx,
                            const oq_rot *rot, int center, int afmt,
                            const uint8_t *w, const void *w_scale, int32_t N, int32_t group,
                            const float *w1, const float *bias, uint16_t *y, int64_t ldy,
                            hipStream_t stream);

/*
 * oq_prepack_w4 -- repack canonical INT4 weights (oq_quant_weight OQ_W4
 * output: codes [N][K/2], scales float32 [N][K/64]) into the tiled FP6
 * layout for OQ_TILED GEMMs.  Values are unchanged (every INT4 code is an
 * exact FP6 E2M3 value).  w_tiled: oq_tiled_bytes(N, K) bytes; w_scale_t:
 * float32 [K/64][N rounded up to 32] (padding columns get scale 0).
 * group must be 64.
 */
int oq_prepack_w4(const uint8_t *w, const float *w_scale, int32_t N, int32_t K, int32_t group,
                  uint8_t *w_tiled, float *w_scale_t, hipStream_t stream);

/*
 * oq_prepack_mx -- repack canonical MXFP4 weights (oq_quant_weight
 * OQ_W_MXFP4 output: codes [N][K/2], E8M0 [N][K/32]) into the tiled MXFP4
 * layout for OQ_MXFP4 | OQ_TILED GEMMs.  Values are unchanged.  w_tiled:
 * oq_tiled_mx_bytes(N, K) bytes; w_e8m0_tiled: a sixteenth of that, 4-byte
 * aligned (padding rows get zero codes and the unit scale 127).
 * K must be a multiple of 128.
 */
int oq_prepack_mx(const uint8_t *w, const uint8_t *w_e8m0, int32_t N, int32_t K,
                  uint8_t *w_tiled, uint8_t *w_e8m0_tiled, hipStream_t stream);

/*
 * Lloyd-Max activation path (OrbitQuant PR #25, "Default changes": Lloyd-Max
 * codes are the method's activation quantizer below 8 bits, with codebooks
 * built per layer width by a Newton solver; CentriQ Sec. 2 "Related work":
 * the codebook comes from the post-rotation marginal; model card
 * FLUX.1-schnell-OrbitQuant-W4A4, "Quantization": codebook lloyd_max,
 * activation normalization epsilon 1e-10).
 *
 * The marginal is that of one coordinate T of a point uniform on the unit
 * sphere S^{d-1}, density proportional to (1 - t^2)^((d-3)/2); tokens are
 * normalised by their RMS, so levels are for U = sqrt(d) T (variance 1).
 */

/*
 * oq_lloyd_max_levels -- host function, no device work.  levels: host
 * float64 [2^bits], ascending: the minimum-MSE quantizer levels of U (every
 * level the mean of U over its cell, every boundary the midpoint of its two
 * levels), solved by Newton's method on those conditions.  d >= 3,
 * bits in [1, 8].  OQ_ERR_UNSUPPORTED if the solve does not converge.
 */
int oq_lloyd_max_levels(int32_t d, int32_t bits, double *levels);

/*
 * oq_lloyd_max_tables -- host function: the stored codebook the kernels use.
 * levels_f16: host uint16 [2^bits], the levels rounded to float16 (RNE);
 * thresholds: host float32 [2^bits - 1], the exact midpoints of adjacent
 * float16 levels (so a code is the nearest stored level).  Copy both to the
 * device for oq_quant_act_lm / oq_gemm_lm.
 */
int oq_lloyd_max_tables(int32_t d, int32_t bits, uint16_t *levels_f16, float *thresholds);

/* bytes of the tiled float16 operand layout for `rows` rows (K % 16 == 0) */
size_t oq_tiled_f16_bytes(int64_t rows, int32_t K);

/*
 * oq_quant_act_lm -- fused (center) -> RPBH rotate -> Lloyd-Max codes.
 *   rho_t = max(RN32(sqrt(S_t / d)), RN32(1e-10)), S_t the float64 sum of
 *   squares of the rotated float32 values; u = RN32(v RN32(1 / rho_t));
 *   code = number of thresholds strictly below u (ties go to the lower level).
 *   scale[t] = rho_t (float32 [M]).
 * tiled == 0: codes are level indices, two per byte (element 2i in bits
 *   3..0) for bits <= 4, else one byte each, rows of ldc_bytes (multiple of 16).
 * tiled != 0: codes receives the float16 levels themselves in the tiled
 *   float16 layout (oq_tiled_f16_bytes(M, d) bytes; ldc_bytes ignored), the
 *   operand oq_gemm_lm takes directly.
 * levels_f16 / thresholds: device copies of oq_lloyd_max_tables' output for
 * the same bits.  rot: RPBH or NULL; d <= 4096.  mean as in oq_quant_act.
 */
int oq_quant_act_lm(const uint16_t *x, int64_t M, int32_t d, int64_t ldx, const oq_rot *rot, int center,
                    int32_t bits, int tiled, const uint16_t *levels_f16, const float *thresholds,
                    void *codes, int64_t ldc_bytes, float *scale, float *mean, hipStream_t stream);

/*
 * oq_prepack_w16 -- dequantize canonical INT4 weights (oq_quant_weight OQ_W4
 * output) to W16[o][k] = RN16(w_scale[o][k / group] * q[o][k]) (the exact
 * product rounded once) in the tiled float16 layout: oq_tiled_f16_bytes(N, K)
 * bytes, padding rows zero.  K % 32 == 0; group a multiple of 32 dividing K.
 */
int oq_prepack_w16(const uint8_t *w, const float *w_scale, int32_t N, int32_t K, int32_t group,
                   uint16_t *w16_tiled, hipStream_t stream);

/*
 * oq_gemm_lm -- Lloyd-Max activations times dequantized weights:
 *   y[t][o] = bf16_RNE( a_scale[t] * sum_k A16[t][k] W16[o][k]
 *                       + mean[t] * w1[o] + bias[o] )
 *   A16 the float16 level of each code; products exact in float32, summed in
 *   float32 on the float16 matrix cores.
 * tiled != 0: qa is oq_quant_act_lm's tiled output (lda_bytes, levels_f16 and
 *   ws unused).  tiled == 0: qa holds level indices as oq_quant_act_lm writes
 *   them for `bits`, rows of lda_bytes; levels_f16 (device) expands them into
 *   ws, which needs oq_workspace_bytes(OQ_OP_GEMM_LM, M, K, N, 0) bytes.
 * w16_tiled from oq_prepack_w16; a_scale float32 [M]; mean and w1 both NULL
 * or both set; bias nullable; y bf16 [M][ldy].  K % 32 == 0.
 * The workgroup shape (256 x 384, 256 x 256 or 256 x 192 outputs) follows M, N and the
 * CU count; OQ_F16_TILE=256x384, 256x256 or 256x192 in the environment forces
 * one.
 * The result does not depend on the shape.
 */
int oq_gemm_lm(int32_t bits, int tiled, const void *qa, int64_t lda_bytes, const float *a_scale, int64_t M,
               int32_t K, const uint16_t *levels_f16, const uint16_t *w16_tiled, int32_t N, const float *mean,
               const float *w1, const float *bias, uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes,
               hipStream_t stream);

/*
 * Asymmetric grouped INT4 weights (CentriQ Sec. 3 Eq. 2: W_g = sigma (Q - z),
 * Q in 0..15, per-(row, group) scale sigma and shift z stored in 16 bits, RTN
 * from the group minimum and maximum; App. B.2: codes stored as Q - 8, the
 * correction C = sigma (z - 8) per row and 64-column group weighted by the
 * group sums p of the activation codes).
 */

/*
 * oq_quant_weight_asym -- offline: rotate each row as oq_quant_weight does,
 * then per group of `group` columns sigma = RNbf16(RN32((max - min) / 15))
 * (1 for a constant group), z = RNbf16(RN32(-min / sigma)),
 * Q = clamp(RNE(RN32(RN32(w / sigma) + z)), 0, 15).
 * codes: Q - 8 as 4-bit two's complement, [N][K/2]; sigma, zero: bfloat16
 * bits [N][K/group]; w1 (nullable) as oq_quant_weight.  K % 64 == 0.
 */
int oq_quant_weight_asym(const float *w, int32_t N, int32_t K, int64_t ldw, const oq_rot *rot, int32_t group,
                         uint8_t *codes, uint16_t *sigma, uint16_t *zero, float *w1, hipStream_t stream);

/*
 * oq_prepack_w4_asym -- repack asymmetric weights for oq_gemm_w4a4_asym:
 * w_tiled (oq_tiled_bytes(N, K) bytes) holds q'/2 for q' = Q - 8 in the tiled
 * FP6 layout; w_scale_t float32 [K/64][N rounded up to 32] = sigma;
 * corr [K/64][N rounded up to 32] pairs of uint32 (8 bytes, 8-byte aligned):
 * C = RN32(sigma RN32(z - 8)) as the three bfloat16 pieces of its truncation
 * split C = c1 + c2 + c3 (each exactly a bfloat16), stored negated as
 * (-c1 | -c2 << 16, -c3); C = -(c1' + c2' + c3') recovers it exactly.
 * (Both tables are group-major so that a row of outputs reads them as one run.)
 * Padding rows get zeros.  group must be 64.
 */
int oq_prepack_w4_asym(const uint8_t *w, const uint16_t *sigma, const uint16_t *zero, int32_t N, int32_t K,
                       int32_t group, uint8_t *w_tiled, float *w_scale_t, uint32_t *corr, hipStream_t stream);

/*
 * oq_quant_act_gsum -- oq_quant_act for afmt OQ_A4 | OQ_TILED or
 * OQ_A6 | OQ_TILED (OQ_SCALE_PCTL allowed), which also writes gsum uint32
 * [d/64][M] (group-major): the sum p of the codes of every 64-wide group
 * (an integer, |p| < 2048) as the operand word of oq_gemm_w4a4_asym, two
 * bfloat16 values whose sum is p exactly: p1 = 8 floor(p / 8) in bits 0-15
 * and p2 = p - p1 (0..7) in bits 16-31.
 * d % 64 == 0, d <= 4096.
 */
int oq_quant_act_gsum(const uint16_t *x, int64_t M, int32_t d, int64_t ldx, const oq_rot *rot, int center, int afmt,
                      void *codes, float *scale, uint32_t *gsum, float *mean, hipStream_t stream);

/*
 * oq_gemm_w4a4_asym -- tiled 4-bit activations times asymmetric weights:
 *   y[t][o] = bf16_RNE( a_scale[t] * sum_g (sigma[o][g] acc_g[t][o]
 *                        - corr[g][o] gsum[g][t]) + mean[t] w1[o] + bias[o] )
 *   acc_g = exact sum over the group of q_a (Q - 8).
 * afmt must be OQ_A4 | OQ_TILED; qa, a_scale, gsum (the packed group sums
 * described above) from oq_quant_act_gsum;
 * w_tiled, w_scale_t, corr from oq_prepack_w4_asym; K % 64 == 0.
 */
int oq_gemm_w4a4_asym(int afmt, const uint8_t *qa, const float *a_scale, const uint32_t *gsum, int64_t M, int32_t K,
                      const uint8_t *w_tiled, const float *w_scale_t, const uint32_t *corr, int32_t N, const float *mean,
                      const float *w1, const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream);

/*
 * Factorised Paley x Sylvester rotation (CentriQ Sec. 4.2 "Rotation", App.
 * B.1): H = (H_m (x) H_b) / sqrt(m b) with H_b Sylvester (b = 2^k) and H_m
 * a Paley matrix (m = 12, 44: type I with q = 11, 43; m = 36: type II with
 * q = 17; m = 1: none), applied as vec(H_b X H_m^T) to the token reshaped
 * column-major to X in R^{b x m}; a row of native width n < m b is centred
 * over its n coordinates and then zero-padded to m b (centering precedes
 * padding).  Descriptor: oq_rot{kind = OQ_ROT_KRON, d = n, block = b,
 * rounds = m, perm = signs = mats = NULL}.  Every output of the rotation,
 * and every code and weight column, has the padded width m b; the GEMMs take
 * K = m b.  oq_rotate, oq_quant_act (integer formats, tiled or not, absmax
 * scale) and oq_quant_weight / oq_quant_weight_asym accept it;
 * oq_linear_fused, group sums, Lloyd-Max codes and the percentile scale do not.
 * Float32 order: un-normalised Sylvester stages on each block, then the
 * m-term sums in increasing c, then one multiply by RN32(1/sqrt(m b)).
 */

/*
 * oq_kron_plan -- host function: the smallest admissible padded width
 * n_pad = m * block >= n with m in {1, 12, 36, 44} and block a power of two
 * of at least 16 (one thread's share of coordinates).  n <= 16384.
 */
int oq_kron_plan(int32_t n, int32_t *m, int32_t *block, int32_t *n_pad);

/*
 * oq_probe_mfma -- measurement helper, not part of the layer: the rate one
 * matrix-core instruction sustains on the calling device at its current clock
 * (a roofline denominator beside the published dense peak, which assumes the
 * top clock).  Launches, on `stream`, two workgroups of four wavefronts per
 * CU that each issue iters x 32 independent instructions of the kind
 * (four accumulator chains, operands in registers, no memory traffic), and
 * returns in *ops the operation count of that launch (2 M N K per
 * instruction); the caller times the launch (for instance with events on the
 * stream) and divides.  sink: device float32 buffer of at least
 * oq_probe_sink_elems() elements (written, values meaningless).  Kinds:
 * OQ_PROBE_FP6 and OQ_PROBE_FP4 (v_mfma_scale_f32_32x32x64_f8f6f4 with both
 * operands FP6 E2M3 / FP4 E2M1, unit scales: the instructions of the tiled
 * INT4 and MXFP4 GEMMs), OQ_PROBE_FP8 (the same instruction on FP8 E4M3),
 * OQ_PROBE_I8 (v_mfma_i32_32x32x32_i8), OQ_PROBE_BF16, OQ_PROBE_F16
 * (v_mfma_f32_32x32x16_bf16 / _f16), and OQ_PROBE_FP6_UPDATE: the tiled INT4
 * GEMM's arithmetic without memory traffic, each FP6 MFMA followed by the 16
 * float32 group-scale updates of the previous tile (8 MFMAs per iteration and
 * wavefront; *ops counts 2 M N K of the MFMAs), the rate the fp32 update
 * leaves to that GEMM.  1 <= iters <= 2^20 (a launch of 2^20 iterations runs
 * for about a second), else OQ_ERR_INVALID_ARG.
 */
enum { OQ_PROBE_FP6 = 1, OQ_PROBE_FP4 = 2, OQ_PROBE_FP8 = 3, OQ_PROBE_I8 = 4, OQ_PROBE_BF16 = 5, OQ_PROBE_F16 = 6,
       OQ_PROBE_FP6_UPDATE = 7 };
int oq_probe_mfma(int kind, int32_t iters, float *sink, double *ops, hipStream_t stream);
size_t oq_probe_sink_elems(void);

enum { OQ_OP_GEMM_W4A8 = 1, OQ_OP_GEMM_W4A4 = 2, OQ_OP_LINEAR = 3, OQ_OP_GEMM_LM = 4 };

/* Scratch bytes a call needs (0 if none).  Pure host function.  For
 * OQ_OP_GEMM_LM, afmt is OQ_TILED for tiled activations, else 0.  For
 * OQ_OP_GEMM_W4A8 (afmt ignored), the optional scratch of the split
 * product, enough for any group size (0 when the product runs in one pass
 * or on the 32 x 32 tile kernel). */
size_t oq_workspace_bytes(int op, int64_t M, int32_t K, int32_t N, int afmt);

#ifdef __cplusplus
}
#endif

#endif /* OQ_H */
