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
// codes to int8 in registers; the operands (and group scales) of the step
// seven ahead are loaded meanwhile into a ring of registers.  After the last
// k step of a group each int32 accumulator is converted and folded into the
// fp32 sum with its column's group scale; the output layout of a 32x32 MFMA
// tile puts column l%32 in lane l, so each lane needs one scale per tile per
// group.  The epilogue takes the workgroup's row scales and means from LDS.
#include "oq_internal.h"

#include <type_traits>

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

  // the workgroup's 128 row scales and means, loaded now and used after the
  // main loop (through LDS: a lane's 16 values lie in 16 different rows)
  float pre_a = 0.f, pre_m = 0.f;
  if (threadIdx.x < 128) {
    int64_t row = (int64_t)blockIdx.y * 128 + threadIdx.x;
    if (row > M - 1) row = M - 1;
    pre_a = a_scale[row];
    if (mean) pre_m = mean[row];
  }
  float w1v[2] = {0.f, 0.f}, bv[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + 32 * j + r32;
    if (col < N) {
      if (mean) w1v[j] = w1[col];
      if (bias) bv[j] = bias[col];
    }
  }

  float F[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) F[i][j][r] = 0.f;

  // k runs in steps of 32 (group / 32 steps per group); the operands of step
  // s + D - 1 are loaded while step s computes, from a ring of D register
  // sets, so that the latency of the plain global loads is covered
  constexpr int D = 8;
  const int SPG = group / 32, S = K / 32;
  typedef typename std::conditional<A_NIB, uint2, uint4>::type RawA;
  RawA ra[D][2];
  uint2 rw[D][2];
  float rs[D][2];  // the group scales of each loaded step's group
  int gl = 0, kl = 0;  // group and step within it of the next load (loads run in step order)
  // Loads are unconditional, from rows and steps clamped into range: rows
  // past M or N only feed outputs that are never stored, and steps past the
  // end are never computed, so no branch splits the copy queue.
  int64_t arc[2];
  int64_t wrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arc[i] = (aok[i] ? arow[i] : M - 1) * lda;
    wrc[i] = (int64_t)(wok[i] ? wrow[i] : N - 1) * (K / 2);
  }
  const float *wsc0 = w_scale + (int64_t)(wok[0] ? wrow[0] : N - 1) * G;
  const float *wsc1 = w_scale + (int64_t)(wok[1] ? wrow[1] : N - 1) * G;
  auto load = [&](int slot, int st) {
    const int k = 32 * (st < S ? st : S - 1) + 16 * half;
    const int gq = gl < G ? gl : G - 1;
    rs[slot][0] = wsc0[gq];
    rs[slot][1] = wsc1[gq];
    if (++kl == SPG) {
      kl = 0;
      ++gl;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (A_NIB) ra[slot][i] = *reinterpret_cast<const uint2 *>(qa + arc[i] + k / 2);
      else ra[slot][i] = *reinterpret_cast<const uint4 *>(qa + arc[i] + k);
      rw[slot][i] = *reinterpret_cast<const uint2 *>(w + wrc[i] + k / 2);
    }
  };
  v16i acc[2][2];
#pragma unroll
  for (int q = 0; q < D - 1; ++q) load(q, q);
  for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      const int st = s0 + q;
      load((q + D - 1) % D, st + D - 1);
      if (st < S) {
        const int kk = st % SPG;
        if (kk == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = (v16i){};
        }
        v4i A[2], B[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if constexpr (A_NIB) {
            A[i] = unpack16(ra[q][i]);
          } else {
            const uint4 p = ra[q][i];
            A[i] = (v4i){(int)p.x, (int)p.y, (int)p.z, (int)p.w};
          }
          B[i] = unpack16(rw[q][i]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[i], B[j], acc[i][j], 0, 0, 0);
        if (kk == SPG - 1) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) F[i][j][r] = __builtin_fmaf(rs[q][j], (float)acc[i][j][r], F[i][j][r]);
        }
      }
    }
  }

  __shared__ float s_alpha[128], s_mean[128];
  if (threadIdx.x < 128) {
    s_alpha[threadIdx.x] = pre_a;
    s_mean[threadIdx.x] = pre_m;
  }
  __syncthreads();
  const int rw0 = (wave >> 1) * 64;  // this wave's first row within the workgroup
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = rw0 + 32 * i + (r >> 2) * 8 + half * 4 + (r & 3);
      const int64_t row = m0 + 32 * i + (r >> 2) * 8 + half * 4 + (r & 3);
      if (row >= M) continue;
      const float al = s_alpha[rl];
      const float mu = s_mean[rl];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + 32 * j + r32;
        if (col >= N) continue;
        float v = al * F[i][j][r];
        if (mean) v = __builtin_fmaf(mu, w1v[j], v);
        if (bias) v = v + bv[j];
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
