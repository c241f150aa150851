// K5: MXFP4 activations x MXFP4 weights on the gfx950 scaled FP4 MFMA.
//
// y[t][o] = bf16( sum_blocks 2^(ea + ew) sum_{k in block} fp4(a) fp4(w) + bias[o] )
// (WUSH review, "Core claim" and Fig. 2 caption: MXFP4 block quantizers with
// G = 32; the element and scale formats are those of the OCP MX v1.0
// specification the review cites.)
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1: lane l holds
// row l%32 and the 32 consecutive k of half l/32 as 16 bytes with element j
// in bits 4j..4j+3, which is exactly the row-major two-codes-per-byte layout
// of the codes, and its E8M0 byte scales those 32 elements.  So operands are
// loaded straight from the code rows; the accumulator carries the whole K.
#include "oq_internal.h"

namespace oq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256)
gemm_mx_kernel(const uint8_t *__restrict__ qa, int64_t lda, const uint8_t *__restrict__ ea, int64_t M,
               int K, const uint8_t *__restrict__ w, const uint8_t *__restrict__ ew, int N,
               const float *__restrict__ bias, uint16_t *__restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * 128 + (wave >> 1) * 64;
  const int n0 = blockIdx.x * 128 + (wave & 1) * 64;
  const int r32 = lane & 31;
  const int half = lane >> 5;
  const int KB = K / 32;

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
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (v16f){};

  for (int k0 = 0; k0 < K; k0 += 64) {
    const int kb = k0 / 32 + half;
    v8i A[2], B[2];
    int sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 p = aok[i] ? *reinterpret_cast<const uint4 *>(qa + arow[i] * lda + kb * 16) : make_uint4(0u, 0u, 0u, 0u);
      A[i] = (v8i){(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
      sa[i] = aok[i] ? (int)ea[arow[i] * KB + kb] : 127;
      const uint4 q = wok[i] ? *reinterpret_cast<const uint4 *>(w + (int64_t)wrow[i] * (K / 2) + kb * 16) : make_uint4(0u, 0u, 0u, 0u);
      B[i] = (v8i){(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      sb[i] = wok[i] ? (int)ew[(int64_t)wrow[i] * KB + kb] : 127;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[i], B[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + 32 * i + (r >> 2) * 8 + half * 4 + (r & 3);
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + 32 * j + r32;
        if (col >= N) continue;
        float v = acc[i][j][r];
        if (bias) v = v + bias[col];
        y[row * ldy + col] = f32_to_bf16_rne(v);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t *qa, int64_t lda_bytes, const uint8_t *a_e8m0, int64_t M, int K,
                          const uint8_t *w, const uint8_t *w_e8m0, int N, const float *bias, uint16_t *y,
                          int64_t ldy, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
  hipLaunchKernelGGL(gemm_mx_kernel, grid, dim3(256), 0, stream, qa, lda_bytes, a_e8m0, M, K, w, w_e8m0, N,
                     bias, y, ldy);
  return hipGetLastError();
}

}  // namespace oq
