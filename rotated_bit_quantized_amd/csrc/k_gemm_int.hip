// K3/K4: integer-coded activations x packed INT4 weights with the fp32
// per-group scale and rank-1 epilogue, gfx950 int8 MFMA.
//
// y[t][o] = bf16( a_scale[t] * sum_g w_scale[o][g] * acc_g[t][o]
//                 + mean[t] * w1[o] + bias[o] )          CentriQ Eq. 5 / Eq. 9
// acc_g = exact int32 sum over the g-th group of input columns
// (CentriQ Sec. 3 Eq. 2: one weight scale per row and group of columns).
//
// Tiling: 256 threads = 4 wavefronts in a 2 x 2 grid; each wavefront owns a
// 64 x 64 output tile = 2 x 2 MFMA 32x32 tiles.  For every 32-deep k step a
// lane feeds v_mfma_i32_32x32x32_i8 with 16 consecutive k of one row
// (lanes 0-31: rows 0-31, k 0-15; lanes 32-63: k 16-31), unpacking 4-bit
// codes to int8 in registers.  After the last k step of a group each int32
// accumulator is converted and folded into the fp32 sum with its column's
// group scale; the output layout of a 32x32 MFMA tile puts column l%32 in
// lane l, so each lane needs one scale per tile per group.
#include "oq_internal.h"

namespace oq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// 8 bytes of 4-bit two's-complement codes -> 16 sign-extended int8, same order
__device__ __forceinline__ v4i unpack16(uint2 p) {
  v4i r;
  const uint32_t src[2] = {p.x, p.y};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t lo = src[h] & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6
    uint32_t hi = (src[h] >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
    // per byte z in [0,15] -> z - 16 [z >= 8] without cross-byte borrow
    lo = ((lo ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
    hi = ((hi ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
    r[2 * h] = (int)__builtin_amdgcn_perm(hi, lo, 0x05010400u);
    r[2 * h + 1] = (int)__builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
  return r;
}

template <bool A_NIB>
__global__ void __launch_bounds__(256)
gemm_int_kernel(const uint8_t *__restrict__ qa, int64_t lda, const float *__restrict__ a_scale,
                int64_t M, int K, const uint8_t *__restrict__ w, const float *__restrict__ w_scale,
                int N, int group, const float *__restrict__ mean, const float *__restrict__ w1,
                const float *__restrict__ bias, uint16_t *__restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * 128 + (wave >> 1) * 64;
  const int n0 = blockIdx.x * 128 + (wave & 1) * 64;
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const int G = K / group;

  int64_t arow[2];
  bool aok[2];
  int wrow[2];
  bool wok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arow[i] = m0 + 32 * i + r32;
    aok[i] = arow[i] < M;
    wrow[i] = n0 + 32 * i + r32;
    wok[i] = wrow[i] < N;
  }

  float F[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) F[i][j][r] = 0.f;

  for (int g = 0; g < G; ++g) {
    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = (v16i){};
    for (int kk = 0; kk < group; kk += 32) {
      const int k = g * group + kk + 16 * half;
      v4i A[2], B[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (A_NIB) {
          const uint2 p = aok[i] ? *reinterpret_cast<const uint2 *>(qa + arow[i] * lda + k / 2) : make_uint2(0u, 0u);
          A[i] = unpack16(p);
        } else {
          const uint4 p = aok[i] ? *reinterpret_cast<const uint4 *>(qa + arow[i] * lda + k) : make_uint4(0u, 0u, 0u, 0u);
          A[i] = (v4i){(int)p.x, (int)p.y, (int)p.z, (int)p.w};
        }
        const uint2 q = wok[i] ? *reinterpret_cast<const uint2 *>(w + (int64_t)wrow[i] * (K / 2) + k / 2) : make_uint2(0u, 0u);
        B[i] = unpack16(q);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[i], B[j], acc[i][j], 0, 0, 0);
    }
    float s[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) s[j] = wok[j] ? w_scale[(int64_t)wrow[j] * G + g] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) F[i][j][r] = __builtin_fmaf(s[j], (float)acc[i][j][r], F[i][j][r]);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + 32 * i + (r >> 2) * 8 + half * 4 + (r & 3);
      if (row >= M) continue;
      const float al = a_scale[row];
      const float mu = mean ? mean[row] : 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + 32 * j + r32;
        if (col >= N) continue;
        float v = al * F[i][j][r];
        if (mean) v = __builtin_fmaf(mu, w1[col], v);
        if (bias) v = v + bias[col];
        y[row * ldy + col] = f32_to_bf16_rne(v);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_int(const void *qa, int64_t lda_bytes, int a_is_nibble, const float *a_scale,
                           int64_t M, int K, const uint8_t *w, const float *w_scale, int N, int group,
                           const float *mean, const float *w1, const float *bias, uint16_t *y,
                           int64_t ldy, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
  if (a_is_nibble)
    hipLaunchKernelGGL((gemm_int_kernel<true>), grid, dim3(256), 0, stream, (const uint8_t *)qa, lda_bytes,
                       a_scale, M, K, w, w_scale, N, group, mean, w1, bias, y, ldy);
  else
    hipLaunchKernelGGL((gemm_int_kernel<false>), grid, dim3(256), 0, stream, (const uint8_t *)qa, lda_bytes,
                       a_scale, M, K, w, w_scale, N, group, mean, w1, bias, y, ldy);
  return hipGetLastError();
}

}  // namespace oq
