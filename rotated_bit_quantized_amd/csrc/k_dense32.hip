// K2: per-32-block dense transform followed by MXFP4 quantization, gfx950.
//
// WUSH review ("Core claim"): every quantization block of 32 coordinates has
// its own transform; activations take T_b, weights its inverse-transpose.
// The quantizer is RTN absmax MXFP4 (E2M1 elements, one E8M0 power-of-two
// scale per 32; OCP MX v1.0 as cited by the review):
//   e = clamp(floor(log2 amax) - 2, -127, 127), element = nearest E2M1 value
//   of v * 2^-e with ties to the even code, saturating at 6, sign kept.
//
// Two kernels.  dense32_kernel (float32 rotated output for oq_rotate, and the
// weight side, which forms T_b^{-T} itself) accumulates the transform in
// float64 and rounds once to float32.  For bf16 x bf16 products the float64
// sum is exact whenever one output's products span at most 32 binades, which
// ordinary activations meet; beyond that its error is at most 2^-47 of the
// sum of the product magnitudes.  Lanes are rows there; the block's matrix is
// staged in LDS as float64 and read as a broadcast.
// dense32_mx_mfma_kernel (the activation MXFP4 path) forms the products on the
// matrix cores and falls back to the same exact float64 sum wherever the
// float32 accumulation could change a code or a block exponent (below).
#include "oq_internal.h"

#pragma clang fp contract(off)

namespace oq {
namespace {

constexpr int BPW = 8;  // blocks per workgroup

__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float m = fabsf(t);
  uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) + (m >= 3.5f) + (m > 5.0f);
  return c | ((__float_as_uint(t) >> 28) & 8u);
}

// Weight side of the pair: T[i][j] = (T_b^{-1})[j][i] from the bfloat16 T_b
// (WUSH review, "Core claim": T_w = T_x^{-T}).  Gauss-Jordan elimination with
// partial pivoting on [T_b | I] in float64, one column of the 32 x 64
// augmented matrix per thread of the 64; the pivot is the first row of
// largest magnitude, read by every thread from a copy of the pivot column.
// Every workgroup that needs block b forms the same inverse (same operations
// in the same order).  T_b is invertible for the transforms this layer is
// built for (cond <= 4); a singular block gives non-finite weights.
__device__ void stage_inverse_transpose(const uint16_t *__restrict__ tb, double *__restrict__ T,
                                        double *__restrict__ aug, double *__restrict__ fcol) {
  const int t = threadIdx.x;  // column of [T_b | I]
  for (int i = 0; i < 32; ++i)
    aug[i * 64 + t] = t < 32 ? (double)__uint_as_float((uint32_t)tb[i * 32 + t] << 16) : (t - 32 == i ? 1.0 : 0.0);
  __syncthreads();
  for (int k = 0; k < 32; ++k) {
    if (t < 32) fcol[t] = aug[t * 64 + k];
    __syncthreads();
    int p = k;
    double best = fabs(fcol[k]);
    for (int i = k + 1; i < 32; ++i) {
      const double a = fabs(fcol[i]);
      if (a > best) {
        best = a;
        p = i;
      }
    }
    const double piv = fcol[p];
    const double rk = aug[p * 64 + t] / piv;  // the new pivot row (old row p), scaled
    const double old_k = aug[k * 64 + t];
    aug[p * 64 + t] = old_k;                   // old row k moves to row p
    aug[k * 64 + t] = rk;
    for (int i = 0; i < 32; ++i) {
      if (i == k) continue;
      const double f = i == p ? fcol[k] : fcol[i];  // factor of the row now at i
      aug[i * 64 + t] = aug[i * 64 + t] - f * rk;
    }
    __syncthreads();
  }
  // T[i][j] = inverse[j][i] = aug[j][32 + i]
  for (int e = t; e < 1024; e += 64) T[e] = aug[(e & 31) * 64 + 32 + (e >> 5)];
  __syncthreads();
}

// IN_F32 selects the weight-side variant: float32 rows, and the matrices are
// the inverse-transposes of the bfloat16 activation transforms.
template <bool IN_F32, bool MX_OUT>
__global__ void __launch_bounds__(64)
dense32_kernel(const void *__restrict__ xin, int64_t M, int d, int64_t ldx, const uint16_t *__restrict__ mats,
               void *__restrict__ out, int64_t ld_out_bytes, uint8_t *__restrict__ e8m0) {
  __shared__ double T[32 * 32];
  __shared__ double aug[IN_F32 ? 32 * 64 : 1];
  __shared__ double fcol[32];
  const int64_t row = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const bool ok = row < M;
  const int nb = d / 32;
  const int b0 = blockIdx.y * BPW;
  const int b1 = min(b0 + BPW, nb);
  for (int b = b0; b < b1; ++b) {
    __syncthreads();
    if (IN_F32) {
      stage_inverse_transpose(mats + (int64_t)b * 1024, T, aug, fcol);
    } else {
      for (int e = threadIdx.x; e < 1024; e += 64)
        T[e] = (double)__uint_as_float((uint32_t)mats[(int64_t)b * 1024 + e] << 16);
      __syncthreads();
    }
    if (!ok) continue;
    double xd[32];
    if (IN_F32) {
      const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(xin) + row * ldx + b * 32);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 p = src[k];
        xd[4 * k] = p.x; xd[4 * k + 1] = p.y; xd[4 * k + 2] = p.z; xd[4 * k + 3] = p.w;
      }
    } else {
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(xin) + row * ldx + b * 32);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 p = src[k];
        const uint32_t wd[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xd[8 * k + 2 * q] = (double)bf16_lo(wd[q]);
          xd[8 * k + 2 * q + 1] = (double)bf16_hi(wd[q]);
        }
      }
    }
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < 32; ++j) acc = __builtin_fma(T[i * 32 + j], xd[j], acc);
      v[i] = (float)acc;
    }
    char *orow = static_cast<char *>(out) + row * ld_out_bytes;
    if (!MX_OUT) {
      float4 *dst = reinterpret_cast<float4 *>(orow) + b * 8;
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
      continue;
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
    const int ef = (int)((__float_as_uint(a) >> 23) & 0xFF);
    const int e = ef == 0 ? -127 : max(ef - 129, -127);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
    uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) wd[i >> 3] |= e2m1_code(v[i] * inv) << (4 * (i & 7));
    *reinterpret_cast<uint4 *>(orow + b * 16) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    e8m0[row * nb + b] = (uint8_t)(e + 127);
  }
}


// Activation path (bf16 in, MXFP4 out) on the matrix cores.  For block b and
// 32 tokens, D = T_b X_b^T by two v_mfma_f32_32x32x16_bf16 over the 32
// inputs: lane l holds token l % 32 and outputs i = 8 (r / 4) + 4 (l / 32)
// + r % 4 in accumulator registers r = 0..15.  A second product
// |T_b| |X_b|^T gives s_i = sum_j |T_ij x_j| (sign bits cleared).
//
// The matrix cores add in float32, so their S'_i may differ from the value the
// codes are defined on, v_i = RN32(sum_j T_ij x_j) (exact products, one
// rounding).  Float32 accumulation of 32 products and an accumulator, with up
// to one ulp per addition (truncation allowed), is off by at most
// 34 * 2^-23 s_i; flushed subnormal products add at most 2^-120.  With the
// RN32 step, s' >= s (1 - 2^-17) and the roundings of S' -+ D below,
// D_i = 2^-17 s'_i + 2^-119 bounds |v_i - S'_i|, and the block's largest,
// D = max_i D_i, bounds that of every output of the block.  An element's code
// is taken from S' when the codes of S'_i - D_i and S'_i + D_i agree (E2M1
// rounding is monotone), the block exponent when the exponents of a' - D and
// a' + D agree (a' = max |S'|); otherwise the value is
// recomputed exactly from the bf16 operands in LDS (float64 sum of the exact
// products in input order, rounded once, as in the float32 path above) and the
// code, or the whole block, is redone from exact values.
//
// Codes come from v_cvt_scalef32_pk_fp4_f32 with scale 2^e, which divides by
// it (exact for a power of two): nearest E2M1 value, ties to the even code,
// saturating, sign kept (checked against the rule above on the device).
// A workgroup covers 4 consecutive blocks (T_b and |T_b| staged in LDS) and
// MXM_TOK tokens, 4 waves of MXM_TPW tiles of 32 tokens; each token's x
// words for the 4 blocks (256 contiguous bytes) are loaded one tile ahead.
// TILED writes the MFMA-tiled MXFP4 layout (see include/oq.h), else row-major
// codes [M][ldc] and E8M0 bytes [M][d/32].
constexpr int MXM_NBG = 4;                     // 32-blocks per workgroup
constexpr int MXM_TPW = 4;                     // 32-token tiles per wave
constexpr int MXM_TOK = 4 * MXM_TPW * 32;      // tokens per workgroup

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  bf16x8_t r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// unbiased E8M0 exponent of a block whose largest magnitude is a >= 0
__device__ __forceinline__ int mx_exponent(float a) {
  const int ef = (int)((__float_as_uint(a) >> 23) & 0xFF);
  return ef == 0 ? -127 : max(ef - 129, -127);
}

// (value in lane l % 32, value in lane l % 32 + 32), in every lane
__device__ __forceinline__ void half_pair(uint32_t v, uint32_t &lo, uint32_t &hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lo = r[0];
  hi = r[1];
}

__device__ __forceinline__ float max_halves(float v) {
  uint32_t a, b;
  half_pair(__float_as_uint(v), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// codes of y[r] / sc for this lane's 16 outputs; word k nibble n is r = 8k + n
__device__ __forceinline__ void pack16(const float (&y)[16], float sc, uint32_t (&w)[2]) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t o = 0u;
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[8 * k], y[8 * k + 1], sc, 0);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[8 * k + 2], y[8 * k + 3], sc, 1);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[8 * k + 4], y[8 * k + 5], sc, 2);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[8 * k + 6], y[8 * k + 7], sc, 3);
    w[k] = o;
  }
}

template <bool TILED>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
dense32_mx_mfma_kernel(const uint16_t *__restrict__ x, int64_t M, int d, int64_t ldx,
                       const uint16_t *__restrict__ mats, uint8_t *__restrict__ codes, int64_t ldc,
                       uint8_t *__restrict__ e8m0) {
  __shared__ __attribute__((aligned(16))) uint16_t Ts[2][MXM_NBG * 1024];  // [0] T_b, [1] |T_b|, row-major
  __shared__ float Vs[4][16 * 64];                                         // per wave: values [r][lane]
  const int nb = d / 32;
  const int b0 = blockIdx.y * MXM_NBG;
  const int nbw = min(MXM_NBG, nb - b0);
  for (int q = threadIdx.x; q < nbw * 128; q += 256) {
    const uint4 w = reinterpret_cast<const uint4 *>(mats + (int64_t)b0 * 1024)[q];
    reinterpret_cast<uint4 *>(Ts[0])[q] = w;
    reinterpret_cast<uint4 *>(Ts[1])[q] =
        make_uint4(w.x & 0x7FFF7FFFu, w.y & 0x7FFF7FFFu, w.z & 0x7FFF7FFFu, w.w & 0x7FFF7FFFu);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, tl = lane & 31;
  const int64_t Mp = (M + 31) / 32 * 32;
  float *vs = Vs[wave];

  // x words of one tile: [block][k-step] = inputs 16 s + 8 h .. + 7 of token tl.
  // Two buffers swap roles from tile to tile (no copy between them, so the
  // compiler's wait for a tile's words never covers the next tile's loads).
  uint4 xA[MXM_NBG][2], xB[MXM_NBG][2];
  auto load_x = [&](int tile, uint4 (&dst)[MXM_NBG][2]) {
    int64_t t = (int64_t)blockIdx.x * MXM_TOK + tile * 32 + tl;
    if (t >= M) t = M - 1;  // rows past the end read the last row; nothing of theirs is stored
    const uint16_t *xr = x + t * ldx + b0 * 32 + 8 * h;
#pragma unroll
    for (int b = 0; b < MXM_NBG; ++b) {
      const int bb = b < nbw ? b : nbw - 1;  // a short last group reloads its last block
#pragma unroll
      for (int s = 0; s < 2; ++s) dst[b][s] = *reinterpret_cast<const uint4 *>(xr + bb * 32 + 16 * s);
    }
  };
  // one tile: prefetch the next tile's words into xn, process xa; false when
  // the tile lies past the last token
  auto tile = [&](int tt, uint4 (&xa)[MXM_NBG][2], uint4 (&xn)[MXM_NBG][2]) -> bool {
    const int64_t tbase = (int64_t)blockIdx.x * MXM_TOK + (wave + 4 * tt) * 32;
    if (tbase >= M) return false;
    // unconditional, so that the compiler's wait for this tile's words never
    // merges with a path without these loads; the last tile reloads its own
    // (cached) rows
    load_x(wave + 4 * (tt + 1 < MXM_TPW ? tt + 1 : tt), xn);
    const int64_t t = tbase + tl;
    const bool valid = t < M;
    uint32_t scw = 0u;  // E8M0 bytes of the group's blocks (tiled layout stores them as one word)

    // the products of block b + 1 are issued before block b is quantized
    f32x16_t acc[2], sig[2];
    auto products = [&](int b, f32x16_t &ac, f32x16_t &sg) {
      ac = f32x16_t{};
      sg = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int off = b * 1024 + tl * 32 + 16 * s + 8 * h;  // A: T_b[i = tl][j = 16 s + 8 h + e]
        const uint4 ta = *reinterpret_cast<const uint4 *>(&Ts[0][off]);
        const uint4 tb = *reinterpret_cast<const uint4 *>(&Ts[1][off]);
        const uint4 xv = xa[b][s];
        const uint4 xb = make_uint4(xv.x & 0x7FFF7FFFu, xv.y & 0x7FFF7FFFu, xv.z & 0x7FFF7FFFu, xv.w & 0x7FFF7FFFu);
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ta), as_bf16x8(xv), ac, 0, 0, 0);
        sg = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(tb), as_bf16x8(xb), sg, 0, 0, 0);
      }
    };
    products(0, acc[0], sig[0]);

#pragma unroll
    for (int b = 0; b < MXM_NBG; ++b) {
      if (b >= nbw) break;
      if (b + 1 < nbw) products(b + 1, acc[(b + 1) & 1], sig[(b + 1) & 1]);
      const int bg = b0 + b;
      const f32x16_t &ac = acc[b & 1];
      float am = 0.f, sm = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        am = fmaxf(am, fabsf(ac[r]));
        sm = fmaxf(sm, sig[b & 1][r]);
      }
      am = max_halves(am);
      sm = max_halves(sm);
      // the block exponent is certain when the exponents of the largest
      // |S'| -+ the largest bound D_i agree; each code when the codes of
      // S'_i -+ D_i agree, D_i = 2^-17 s_i + 2^-119 its own bound
      const float da = __builtin_fmaf(sm, 0x1p-17f, 0x1p-119f);
      int e = mx_exponent(am);
      // tiny blocks (e < -100, e.g. all zero) always take the exact path
      const bool blk = e < -100 || mx_exponent(fmaxf(am - da, 0.f)) != mx_exponent(am + da);
      float sc = __uint_as_float((uint32_t)(127 + max(e, -126)) << 23);  // 2^e, normal
      float dl[16], dh[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float di = __builtin_fmaf(sig[b & 1][r], 0x1p-17f, 0x1p-119f);
        dl[r] = ac[r] - di;
        dh[r] = ac[r] + di;
      }
      // codes of S' - D and S' + D; word k nibble n is register r = 8 k + n
      uint32_t wl[2], wh[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int r = 8 * k;
        uint32_t ol = 0u, oh = 0u;
        ol = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ol, dl[r], dl[r + 1], sc, 0);
        oh = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(oh, dh[r], dh[r + 1], sc, 0);
        ol = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ol, dl[r + 2], dl[r + 3], sc, 1);
        oh = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(oh, dh[r + 2], dh[r + 3], sc, 1);
        ol = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ol, dl[r + 4], dl[r + 5], sc, 2);
        oh = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(oh, dh[r + 4], dh[r + 5], sc, 2);
        ol = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ol, dl[r + 6], dl[r + 7], sc, 3);
        oh = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(oh, dh[r + 6], dh[r + 7], sc, 3);
        wl[k] = ol;
        wh[k] = oh;
      }
      const uint32_t d0 = wl[0] ^ wh[0], d1 = wl[1] ^ wh[1];
      const bool need = valid && (blk || (d0 | d1) != 0u);
      if (__ballot(need) != 0ull) {
        // all 32 inputs of the token: this lane's half and its partner's
        uint4 xin[4];  // inputs 8 q .. 8 q + 7
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint4 o = xa[b][s];
          const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
          uint32_t pw[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t lw, hw;
            half_pair(ow[k], lw, hw);
            pw[k] = h ? lw : hw;
          }
          const uint4 p = make_uint4(pw[0], pw[1], pw[2], pw[3]);
          xin[2 * s] = h ? p : o;
          xin[2 * s + 1] = h ? o : p;
        }
        // exact value of output r of this lane's token (r may differ from
        // lane to lane): four float64 partial sums of the exact products,
        // each exact, as is their total, whenever the products span at most
        // 32 binades; rounded once to float32
        auto exact = [&](int r) -> float {
          const int i = 8 * (r >> 2) + 4 * h + (r & 3);
          const uint4 *trow = reinterpret_cast<const uint4 *>(&Ts[0][b * 1024 + i * 32]);
          double sp[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 tw = trow[q];
            const uint32_t tws[4] = {tw.x, tw.y, tw.z, tw.w};
            const uint32_t xws[4] = {xin[q].x, xin[q].y, xin[q].z, xin[q].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              sp[k] = __builtin_fma((double)bf16_lo(tws[k]), (double)bf16_lo(xws[k]), sp[k]);
              sp[k] = __builtin_fma((double)bf16_hi(tws[k]), (double)bf16_hi(xws[k]), sp[k]);
            }
          }
          return (float)((sp[0] + sp[1]) + (sp[2] + sp[3]));
        };
        // certain exponent: redo the outputs whose two codes differ and
        // patch their nibbles, one flagged output per lane per pass (the
        // lanes' outputs differ; a single pass is the common case)
        uint32_t fm = 0u;  // bit r: nibble r of the two code words differs
        if (valid && !blk) {
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            fm |= (((d0 >> (4 * n)) & 0xFu) != 0u ? 1u : 0u) << n;
            fm |= (((d1 >> (4 * n)) & 0xFu) != 0u ? 1u : 0u) << (n + 8);
          }
        }
        while (__ballot(fm != 0u) != 0ull) {
          if (fm != 0u) {
            const int r = __builtin_ctz(fm);
            fm &= fm - 1u;
            const float ve = exact(r);
            const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, ve, ve, sc, 0) & 0xFu;
            const int sh = 4 * (r & 7);
            const uint32_t keep = ~(0xFu << sh);
            if (r < 8)
              wl[0] = (wl[0] & keep) | (c << sh);
            else
              wl[1] = (wl[1] & keep) | (c << sh);
          }
        }
        // uncertain exponent (both lanes of the token): redo all 32 outputs,
        // take the exponent from them, recode the block
        const bool bl = valid && blk;
        if (__ballot(bl) != 0ull) {
#pragma unroll 1
          for (int r = 0; r < 16; ++r)
            if (bl) vs[r * 64 + lane] = exact(r);
          float ve[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) ve[r] = vs[r * 64 + lane];  // meaningful where bl
          float ae = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) ae = fmaxf(ae, fabsf(ve[r]));
          ae = max_halves(ae);
          const int eb = mx_exponent(ae);
          float mul = 1.0f, sb = __uint_as_float((uint32_t)(127 + max(eb, -126)) << 23);
          if (eb < -126) {  // 2^-127 is not a normal scale: multiply by 2^127 (exact) instead
            mul = 0x1p127f;
            sb = 1.0f;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) ve[r] *= mul;
          uint32_t wb[2];
          pack16(ve, sb, wb);
          if (bl) {
            e = eb;
            wl[0] = wb[0];
            wl[1] = wb[1];
          }
        }
      }
      // this lane has bytes 4 q + 2 h, 4 q + 2 h + 1 of the token's 16; the
      // lane pair swaps halves so that lane h stores bytes 8 h .. 8 h + 7
      uint32_t p0, p1;
      half_pair(h ? wl[0] : wl[1], p0, p1);
      const uint32_t rcv = h ? p0 : p1;
      const uint2 o = h ? make_uint2((rcv & 0xFFFFu) | (wl[1] << 16), (rcv >> 16) | (wl[1] & 0xFFFF0000u))
                        : make_uint2((wl[0] & 0xFFFFu) | (rcv << 16), (wl[0] >> 16) | (rcv & 0xFFFF0000u));
      if (valid) {
        if (TILED) {
          uint8_t *tile = codes + ((t >> 5) * (d >> 6) + (bg >> 1)) * 1024;
          *reinterpret_cast<uint2 *>(tile + 16 * (32 * (bg & 1) + tl) + 8 * h) = o;
        } else {
          *reinterpret_cast<uint2 *>(codes + t * ldc + bg * 16 + 8 * h) = o;
          if (h == 0) e8m0[t * nb + bg] = (uint8_t)(e + 127);
        }
      }
      scw |= (uint32_t)(e + 127) << (8 * b);
    }
    if (TILED && valid && h == 0)  // the group is 4 aligned blocks when TILED (d % 128 == 0)
      *reinterpret_cast<uint32_t *>(e8m0 + ((int64_t)(b0 >> 2) * Mp + t) * 4) = scw;
    return true;
  };
  static_assert(MXM_TPW % 2 == 0, "tiles are taken in pairs");
  load_x(wave, xA);
  for (int tt = 0; tt < MXM_TPW; tt += 2) {
    if (!tile(tt, xA, xB)) break;
    if (!tile(tt + 1, xB, xA)) break;
  }
}

template <bool IN_F32, bool MX_OUT>
hipError_t launch(const void *x, int64_t M, int d, int64_t ldx, const uint16_t *mats, void *out,
                  int64_t ld_out_bytes, uint8_t *e8m0, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int nb = d / 32;
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)((nb + BPW - 1) / BPW));
  hipLaunchKernelGGL((dense32_kernel<IN_F32, MX_OUT>), grid, dim3(64), 0, stream, x, M, d, ldx, mats, out,
                     ld_out_bytes, e8m0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense32(const uint16_t *x, int64_t M, int d, int64_t ldx, const uint16_t *mats, int mx_out,
                          void *out, int64_t ld_out_bytes, uint8_t *e8m0, hipStream_t stream) {
  if (mx_out) {
    if (M == 0) return hipSuccess;
    const int nb = d / 32;
    dim3 grid((unsigned)((M + MXM_TOK - 1) / MXM_TOK), (unsigned)((nb + MXM_NBG - 1) / MXM_NBG));
    if (mx_out == 2)
      hipLaunchKernelGGL(dense32_mx_mfma_kernel<true>, grid, dim3(256), 0, stream, x, M, d, ldx, mats,
                         static_cast<uint8_t *>(out), ld_out_bytes, e8m0);
    else
      hipLaunchKernelGGL(dense32_mx_mfma_kernel<false>, grid, dim3(256), 0, stream, x, M, d, ldx, mats,
                         static_cast<uint8_t *>(out), ld_out_bytes, e8m0);
    return hipGetLastError();
  }
  return launch<false, false>(x, M, d, ldx, mats, out, ld_out_bytes, e8m0, stream);
}

hipError_t launch_weight_dense32(const float *w, int N, int K, int64_t ldw, const uint16_t *mats,
                                 uint8_t *codes, uint8_t *e8m0, float *w1, hipStream_t stream) {
  (void)w1;
  return launch<true, true>(w, N, K, ldw, mats, codes, K / 2, e8m0, stream);
}

}  // namespace oq
