// K1: per-token (center) -> RPBH rotation -> absmax quantize -> pack, gfx950.
//
// Computes, for every token row x_t (bfloat16):
//   CentriQ Sec. 4.2 Eq. 4: m_t = mean of the row, x^c = x - m_t (optional);
//   OrbitQuant PR #25 ("Default changes", "Runtime work"): one or two RPBH
//     rounds, each a signed gather over the whole width followed by a
//     normalised Sylvester-Hadamard transform of every block of h coordinates;
//   CentriQ Sec. 3 Eq. 1: symmetric per-token absmax codes with one scale.
//
// Layout: one workgroup walks token rows; thread t owns the 16 consecutive
// coordinates [16t, 16t+16) of the row, so a block of h coordinates is held
// by h/16 consecutive lanes of one wavefront (h <= 1024 = 64 lanes x 16).
// The gather of each round reads the previous values from LDS at the
// permuted positions; the first four Hadamard stages (strides 1..8) run in
// registers, the remaining ones exchange values between lanes.  Float32
// results follow the canonical order: strides 1, 2, 4, ... each butterfly
// rounded once, then one multiply by RN32(1/sqrt h).
#include "oq_internal.h"

#pragma clang fp contract(off)

namespace oq {
namespace {

constexpr int E = 16;  // coordinates per thread

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// In-register butterflies over the 16 coordinates of one thread (strides 1..8).
__device__ __forceinline__ void fwht16(float (&u)[E]) {
#pragma unroll
  for (int s = 1; s < E; s <<= 1) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if ((j & s) == 0) {
        const float a = u[j], b = u[j + s];
        u[j] = a + b;
        u[j + s] = a - b;
      }
    }
  }
}

// IN_F32: rows are float32 (offline weight fold) instead of bfloat16.
// MODE OUT_W4G: symmetric INT4 per group of `group` coordinates (weights),
//   scale_out [M][d/group]; mean_out, if set, receives the float64 row sum of
//   the input rounded to float32 (w1 = W 1).
// MODE OUT_W4A: asymmetric INT4 per group (CentriQ Sec. 3 Eq. 2, RTN from the
//   group's minimum and maximum): sigma = RNbf16(RN32((max - min) / 15)) (1
//   for a constant group), z = RNbf16(RN32(-min / sigma)), codes
//   Q = clamp(RNE(RN32(RN32(w / sigma) + z)), 0, 15) stored as Q - 8;
//   sigma bits to scale_out (as uint16), z bits to zero_out.
// KRON: the factorised rotation (H_m (x) H_h) / sqrt(d) of CentriQ Sec. 4.2
// "Rotation" / App. B.1 instead of RPBH rounds (ROUNDS must be 1): the row
// holds din native coordinates, centred over those, then zero-padded to d =
// km h; the Sylvester factor runs on every block of h (un-normalised, the
// usual stages), then out[c' h + r] = sum_c H_m[c'][c] u[c h + r] in
// increasing c, then one multiply by c_h = RN32(1 / sqrt(d)).
template <int ROUNDS, int MODE, bool IN_F32, bool KRON = false>
__global__ void __launch_bounds__(1024)
rpbh_quant_kernel(const void *__restrict__ xin, int64_t M, int d, int64_t ldx,
                  const int32_t *__restrict__ perm, const int8_t *__restrict__ signs,
                  int h, float c_h, int center, float *__restrict__ mean_out,
                  int qmax, void *__restrict__ out, int64_t ld_out_bytes,
                  float *__restrict__ scale_out, int group, uint16_t *__restrict__ zero_out,
                  int din, int km) {
  static_assert(!KRON || ROUNDS == 1, "the Kronecker rotation is one transform");
  extern __shared__ float lds[];
  float *buf0 = lds;                      // [d]
  float *buf1 = lds + (ROUNDS == 2 ? d : 0);
  float *red = lds + (ROUNDS == 2 ? 2 * d : (ROUNDS == 1 ? d : 0));  // [16] floats
  double *redd = reinterpret_cast<double *>(red + 16);                // [16] doubles

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int nwaves = blockDim.x >> 6;
  const int nact = d / E;                 // threads that own coordinates
  const bool act = t < nact;
  const int base = t * E;

  // per-thread gather offsets and sign masks, loaded once per workgroup
  int off[ROUNDS > 0 ? ROUNDS : 1][E];
  uint32_t smask[ROUNDS > 0 ? ROUNDS : 1][E];
  const bool ldin = act && base < din;  // coordinates of the input row (the rest is padding)
  uint64_t hmask = 0;
  if constexpr (KRON) {
    if (act) hmask = paley_row_mask(km, base / h);
  }
#pragma unroll
  for (int r = 0; r < (KRON ? 0 : ROUNDS); ++r) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = act ? base + j : 0;
      off[r][j] = perm[(int64_t)r * d + i];
      smask[r][j] = signs[(int64_t)r * d + i] < 0 ? 0x80000000u : 0u;
    }
  }

  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    __syncthreads();  // previous row's LDS readers are done
    float v[E];
    if (ldin && IN_F32) {
      const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(xin) + row * ldx + base);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 p = src[k];
        v[4 * k] = p.x; v[4 * k + 1] = p.y; v[4 * k + 2] = p.z; v[4 * k + 3] = p.w;
      }
    } else if (ldin) {
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(xin) + row * ldx + base);
      const uint4 p0 = src[0], p1 = src[1];
      const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[2 * k] = bf16_lo(w[k]);
        v[2 * k + 1] = bf16_hi(w[k]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = 0.f;
    }

    if (MODE == OUT_W4G || MODE == OUT_W4A) {
      if (mean_out) {  // w1 = row sum of the unrotated weight, float64 then RN32
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < E; ++j) s += (double)v[j];
        s = wave_sum(s);
        if (lane == 0) redd[wave] = s;
        __syncthreads();
        double tot = 0.0;
        for (int w = 0; w < nwaves; ++w) tot += redd[w];
        if (t == 0) mean_out[row] = (float)tot;
      }
    } else if (center) {
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < E; ++j) s += (double)v[j];
      s = wave_sum(s);
      if (lane == 0) redd[wave] = s;
      __syncthreads();
      double tot = 0.0;
      for (int w = 0; w < nwaves; ++w) tot += redd[w];
      const float m = (float)(tot / (double)din);
      if (ldin) {  // padding stays zero: centering precedes padding
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = v[j] - m;
      }
      if (t == 0) mean_out[row] = m;
    }

    if constexpr (KRON) {
      fwht16(v);
      const int hw = h < 1024 ? h : 1024;
      for (int s = E; s < hw; s <<= 1) {
        const int m = s / E;
        const float sg = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float p = __shfl_xor(v[j], m);
          v[j] = __builtin_fmaf(v[j], sg, p);
        }
      }
      // strides of 1024 and more pair coordinates held by different
      // wavefronts: exchange through LDS, same butterflies
      for (int s = 1024; s < h; s <<= 1) {
        if (act) {
          float4 *dst = reinterpret_cast<float4 *>(buf0 + base);
#pragma unroll
          for (int k = 0; k < 4; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
        }
        __syncthreads();
        if (act) {
          const bool hi = (base & s) != 0;
          const float4 *src = reinterpret_cast<const float4 *>(buf0 + (base ^ s));
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float4 pp = src[k];
            const float p4[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * k + e] = hi ? p4[e] - v[4 * k + e] : v[4 * k + e] + p4[e];
          }
        }
        __syncthreads();
      }
      if (act) {
        float4 *dst = reinterpret_cast<float4 *>(buf0 + base);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
      }
      __syncthreads();
      if (act) {
        // this thread's 16 outputs share the block c' = base / h and sit at
        // offsets r0 .. r0 + 15 of it
        const int r0 = base % h;
        float acc[E];
        for (int c = 0; c < km; ++c) {
          const float4 *src = reinterpret_cast<const float4 *>(buf0 + c * h + r0);
          const bool neg = (hmask >> c) & 1;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float4 pp = src[k];
            const float p4[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float t = neg ? -p4[e] : p4[e];
              acc[4 * k + e] = c == 0 ? t : acc[4 * k + e] + t;
            }
          }
        }
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = acc[j] * c_h;
      }
    }
#pragma unroll
    for (int r = 0; r < (KRON ? 0 : ROUNDS); ++r) {
      float *buf = (r == 0) ? buf0 : buf1;
      if (act) {
        float4 *dst = reinterpret_cast<float4 *>(buf + base);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = __uint_as_float(__float_as_uint(buf[off[r][j]]) ^ smask[r][j]);
      fwht16(v);
      for (int s = E; s < h; s <<= 1) {
        const int m = s / E;
        const float sg = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float p = __shfl_xor(v[j], m);
          // low partner: a + b; high partner: b_low - a_high, one rounding
          v[j] = __builtin_fmaf(v[j], sg, p);
        }
      }
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = v[j] * c_h;
    }

    if (MODE == OUT_F32) {
      if (act && out) {
        float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<char *>(out) + row * ld_out_bytes) + t * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
      }
      continue;
    }

    if (MODE == OUT_W4A) {
      // groups of `group` coordinates = group/16 consecutive lanes
      float mn = v[0], mx = v[0];
#pragma unroll
      for (int j = 1; j < E; ++j) {
        mn = fminf(mn, v[j]);
        mx = fmaxf(mx, v[j]);
      }
      for (int m = 1; m < group / E; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
      }
      const float r = mx - mn;
      const uint16_t sb = r > 0.f ? f32_to_bf16_rne(__fdiv_rn(r, 15.0f)) : (uint16_t)0x3F80;  // 1.0
      const float sig = __uint_as_float((uint32_t)sb << 16);
      const uint16_t zb = f32_to_bf16_rne(__fdiv_rn(-mn, sig));
      const float z = __uint_as_float((uint32_t)zb << 16);
      if (!act) continue;
      if ((base % group) == 0) {
        const int64_t gi = row * (d / group) + base / group;
        reinterpret_cast<uint16_t *>(scale_out)[gi] = sb;
        zero_out[gi] = zb;
      }
      uint32_t wd[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float tq = __builtin_rintf(__fdiv_rn(v[j], sig) + z);
        const int q = (int)fminf(fmaxf(tq, 0.0f), 15.0f) - 8;
        wd[j >> 3] |= (uint32_t)(q & 0xF) << (4 * (j & 7));
      }
      char *orow = reinterpret_cast<char *>(out) + row * ld_out_bytes;
      *reinterpret_cast<uint2 *>(orow + base / 2) = make_uint2(wd[0], wd[1]);
      continue;
    }

    if (MODE == OUT_W4G) {
      // groups of `group` coordinates = group/16 consecutive lanes
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) a = fmaxf(a, fabsf(v[j]));
      for (int m = 1; m < group / E; m <<= 1) a = fmaxf(a, __shfl_xor(a, m));
      a = fmaxf(a, 1e-10f);
      const float sw = __fdiv_rn(a, 7.0f);
      const float inv = __fdiv_rn(7.0f, a);
      if (!act) continue;
      if ((base % group) == 0) scale_out[row * (d / group) + base / group] = sw;
      uint32_t wd[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float tq = __builtin_rintf(v[j] * inv);
        const int q = (int)fminf(fmaxf(tq, -7.0f), 7.0f);
        wd[j >> 3] |= (uint32_t)(q & 0xF) << (4 * (j & 7));
      }
      char *orow = reinterpret_cast<char *>(out) + row * ld_out_bytes;
      *reinterpret_cast<uint2 *>(orow + base / 2) = make_uint2(wd[0], wd[1]);
      continue;
    }

    float a = 0.f;
    if (act) {  // idle lanes hold rotated copies of other coordinates
#pragma unroll
      for (int j = 0; j < E; ++j) a = fmaxf(a, fabsf(v[j]));
    }
    a = wave_max(a);
    if (lane == 0) red[wave] = a;
    __syncthreads();
    a = 0.f;
    for (int w = 0; w < nwaves; ++w) a = fmaxf(a, red[w]);
    a = fmaxf(a, 1e-10f);
    const float fq = (float)qmax;
    const float alpha = __fdiv_rn(a, fq);
    const float inv = __fdiv_rn(fq, a);
    if (t == 0) scale_out[row] = alpha;
    if (!act) continue;

    int q[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const float tq = __builtin_rintf(v[j] * inv);
      q[j] = (int)fminf(fmaxf(tq, -fq), fq);
    }
    if (MODE == OUT_FP6 || MODE == OUT_FP6X2) {
      // tiled layout (see k_gemm_fp6.hip): this thread's 16 values are the
      // first or second 96 bits of the 192-bit string of (row, k-half), whose
      // bytes 0..15 sit at tile + 16 l and bytes 16..23 at tile + 1024 + 8 l
      const int kg = base >> 6, hf = (base >> 5) & 1, j0 = base & 31;
      const int l = 32 * hf + (int)(row & 31);
      uint8_t *tile = static_cast<uint8_t *>(out) + ((row >> 5) * (d >> 6) + kg) * 1536;
      const int64_t pstride = tiled_bytes(M, d);
#pragma unroll
      for (int p = 0; p < (MODE == OUT_FP6X2 ? 2 : 1); ++p) {
        uint32_t c[E];
#pragma unroll
        for (int j = 0; j < E; ++j)
          c[j] = fp6_e2m3_of_int(MODE == OUT_FP6 ? q[j] : (p == 0 ? (q[j] >> 3) : (q[j] & 7)));
        uint64_t lo = 0;
#pragma unroll
        for (int j = 0; j < 10; ++j) lo |= (uint64_t)c[j] << (6 * j);
        lo |= (uint64_t)(c[10] & 0xFu) << 60;
        const uint32_t w0 = (uint32_t)lo, w1 = (uint32_t)(lo >> 32);
        const uint32_t w2 = (c[10] >> 4) | (c[11] << 2) | (c[12] << 8) | (c[13] << 14) | (c[14] << 20) | (c[15] << 26);
        uint8_t *tp = tile + p * pstride;
        if (j0 == 0) {
          *reinterpret_cast<uint2 *>(tp + 16 * l) = make_uint2(w0, w1);
          *reinterpret_cast<uint32_t *>(tp + 16 * l + 8) = w2;
        } else {
          *reinterpret_cast<uint32_t *>(tp + 16 * l + 12) = w0;
          *reinterpret_cast<uint2 *>(tp + 1024 + 8 * l) = make_uint2(w1, w2);
        }
      }
      continue;
    }
    char *orow = reinterpret_cast<char *>(out) + row * ld_out_bytes;
    if (MODE == OUT_I8) {
      uint32_t wd[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        wd[k] = (uint32_t)(q[4 * k] & 0xFF) | ((uint32_t)(q[4 * k + 1] & 0xFF) << 8) |
                ((uint32_t)(q[4 * k + 2] & 0xFF) << 16) | ((uint32_t)(q[4 * k + 3] & 0xFF) << 24);
      *reinterpret_cast<uint4 *>(orow + base) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    } else {  // OUT_I4
      uint32_t wd[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < E; ++j) wd[j >> 3] |= (uint32_t)(q[j] & 0xF) << (4 * (j & 7));
      *reinterpret_cast<uint2 *>(orow + base / 2) = make_uint2(wd[0], wd[1]);
    }
  }
}

template <int ROUNDS, int MODE, bool IN_F32, bool KRON = false>
hipError_t launch_t(const void *x, int64_t M, int d, int64_t ldx, const RotArgs &rot,
                    int center, float *mean, int qmax, void *out, int64_t ld_out_bytes,
                    float *scale, int group, hipStream_t stream, uint16_t *zero = nullptr, int din = -1) {
  const int nact = d / E;
  const int threads = ((nact + 63) / 64) * 64;
  const size_t lds = sizeof(float) * ((size_t)ROUNDS * d + 16) + sizeof(double) * 16;
  // enough workgroups to cover the chip several times; each walks rows
  int64_t grid = M < 4096 ? M : 4096;
  if (grid < 1) grid = 1;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void *)rpbh_quant_kernel<ROUNDS, MODE, IN_F32, KRON>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((rpbh_quant_kernel<ROUNDS, MODE, IN_F32, KRON>), dim3((unsigned)grid), dim3(threads), lds, stream,
                     x, M, d, ldx, rot.perm, rot.signs, rot.block, rot.c_h, center, mean, qmax, out,
                     ld_out_bytes, scale, group, zero, din < 0 ? d : din, KRON ? rot.kron_m : 0);
  return hipGetLastError();
}

template <int ROUNDS>
hipError_t launch_mode(int mode, const uint16_t *x, int64_t M, int d, int64_t ldx, const RotArgs &rot,
                       int center, float *mean, int qmax, void *out, int64_t ld_out_bytes,
                       float *scale, hipStream_t stream) {
  switch (mode) {
    case OUT_F32: return launch_t<ROUNDS, OUT_F32, false>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream);
    case OUT_I8: return launch_t<ROUNDS, OUT_I8, false>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream);
    case OUT_I4: return launch_t<ROUNDS, OUT_I4, false>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream);
    case OUT_FP6: return launch_t<ROUNDS, OUT_FP6, false>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream);
    case OUT_FP6X2: return launch_t<ROUNDS, OUT_FP6X2, false>(x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_weight_rpbh(const float *w, int N, int K, int64_t ldw, const RotArgs &rot, int group,
                              uint8_t *codes, float *scales, float *w1, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (rot.kron_m) {
    const int Kp = rot_out_width(rot, K);
    return launch_t<1, OUT_W4G, true, true>(w, N, Kp, ldw, rot, 0, w1, 7, codes, Kp / 2, scales, group, stream, nullptr,
                                            K);
  }
  switch (rot.rounds) {
    case 0: return launch_t<0, OUT_W4G, true>(w, N, K, ldw, rot, 0, w1, 7, codes, K / 2, scales, group, stream);
    case 1: return launch_t<1, OUT_W4G, true>(w, N, K, ldw, rot, 0, w1, 7, codes, K / 2, scales, group, stream);
    case 2: return launch_t<2, OUT_W4G, true>(w, N, K, ldw, rot, 0, w1, 7, codes, K / 2, scales, group, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_weight_rpbh_asym(const float *w, int N, int K, int64_t ldw, const RotArgs &rot, int group,
                                   uint8_t *codes, uint16_t *sigma, uint16_t *zero, float *w1, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  float *sg = reinterpret_cast<float *>(sigma);  // carried as the scale pointer, written as uint16
  if (rot.kron_m) {
    const int Kp = rot_out_width(rot, K);
    return launch_t<1, OUT_W4A, true, true>(w, N, Kp, ldw, rot, 0, w1, 0, codes, Kp / 2, sg, group, stream, zero, K);
  }
  switch (rot.rounds) {
    case 0: return launch_t<0, OUT_W4A, true>(w, N, K, ldw, rot, 0, w1, 0, codes, K / 2, sg, group, stream, zero);
    case 1: return launch_t<1, OUT_W4A, true>(w, N, K, ldw, rot, 0, w1, 0, codes, K / 2, sg, group, stream, zero);
    case 2: return launch_t<2, OUT_W4A, true>(w, N, K, ldw, rot, 0, w1, 0, codes, K / 2, sg, group, stream, zero);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rpbh_quant(const uint16_t *x, int64_t M, int d, int64_t ldx, const RotArgs &rot,
                             int center, float *mean, int out_mode, int qmax, void *out,
                             int64_t ld_out_bytes, float *scale, hipStream_t stream, const PctlArgs *pctl,
                             const LmArgs *lm, uint32_t *gsum) {
  if (M == 0) return hipSuccess;
  if (rot.kron_m) {
    // the Kronecker rotation runs at the padded width: on the wave kernel for
    // the shapes it covers, else on the workgroup kernel
    if (pctl || lm || gsum) return hipErrorInvalidValue;
    const bool wave_mode = out_mode == OUT_F32 || out_mode == OUT_I8 || out_mode == OUT_I4 || out_mode == OUT_FP6 ||
                           out_mode == OUT_FP6X2;
    if (wave_mode && rpbh_wave_kron_supported(rot.kron_m, rot.block, d))
      return launch_rpbh_wave_kron(x, M, d, ldx, rot, center, mean, out_mode, qmax, out, ld_out_bytes, scale, stream);
    const int dp = rot_out_width(rot, d);
    switch (out_mode) {
      case OUT_F32: return launch_t<1, OUT_F32, false, true>(x, M, dp, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream, nullptr, d);
      case OUT_I8: return launch_t<1, OUT_I8, false, true>(x, M, dp, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream, nullptr, d);
      case OUT_I4: return launch_t<1, OUT_I4, false, true>(x, M, dp, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream, nullptr, d);
      case OUT_FP6: return launch_t<1, OUT_FP6, false, true>(x, M, dp, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream, nullptr, d);
      case OUT_FP6X2: return launch_t<1, OUT_FP6X2, false, true>(x, M, dp, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, 0, stream, nullptr, d);
    }
    return hipErrorInvalidValue;
  }
  if (rpbh_wave_supported(d))
    return launch_rpbh_wave(x, M, d, ldx, rot, center, mean, out_mode, qmax, out, ld_out_bytes, scale, stream, pctl, lm,
                            gsum);
  // the percentile range, the Lloyd-Max codes and the group sums exist in the wave kernel only
  if (pctl || lm || gsum || out_mode >= OUT_LM4) return hipErrorInvalidValue;
  switch (rot.rounds) {
    case 0: return launch_mode<0>(out_mode, x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, stream);
    case 1: return launch_mode<1>(out_mode, x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, stream);
    case 2: return launch_mode<2>(out_mode, x, M, d, ldx, rot, center, mean, qmax, out, ld_out_bytes, scale, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace oq
