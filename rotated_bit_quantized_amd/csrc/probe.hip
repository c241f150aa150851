// Measured roofline denominators: a stream of independent matrix-core
// instructions of one kind on every SIMD of the device, with nothing else to
// do, so that timing one launch gives the rate the instruction sustains on the
// calling device at its current clock (the published dense peaks assume the
// top clock).  Each wavefront keeps four accumulator chains, so every
// instruction's result is needed four instructions later and the matrix core
// never waits on a dependence.  Operands are fixed register values; the
// accumulators are written to `sink` at the end so that nothing is removed.
#include "oq_internal.h"

namespace oq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int PROBE_CHAINS = 4;
constexpr int PROBE_UNROLL = 8;  // instructions per chain per loop iteration

// The FP6 GEMM's own arithmetic without memory: per step one FP6 MFMA with
// a zero accumulator (the exact group sum of a 32 x 32 tile) and the 16
// float32 updates F += s * sum of the previous tile's result, eight tiles per
// group, as the tiled INT4 GEMM's main loop issues them; iters groups.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fp6_update_probe_kernel(int iters, float *__restrict__ sink) {
  const int t = threadIdx.x;
  float F[8][16];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) F[i][e] = 0.f;
  v8i A[4], B[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) A[i] = (v8i){t, 0x11111111 * i, 0x02020202, 0x03030303, 0x04040404, 0x05050505, 0, 0};
#pragma unroll
  for (int j = 0; j < 2; ++j) B[j] = (v8i){0x01010101, t + j, 0x02020202, 0x01010101, 0x03030303, 0x01010101, 0, 0};
  const float s0 = 1.0f + 1e-3f * (t & 63), s1 = 1.0f - 1e-3f * (t & 63);
  for (int it = 0; it < iters; ++it) {
    v16f dprev = (v16f){};
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int i = tt % 4, j = tt / 4;
      const v16f dt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[i], B[j], (v16f){}, 2, 2, 0, 127, 0, 127);
      __builtin_amdgcn_sched_barrier(0);
      if (tt > 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) F[tt - 1][e] = __builtin_fmaf(j ? s1 : s0, dprev[e], F[tt - 1][e]);
      }
      __builtin_amdgcn_sched_barrier(0);
      dprev = dt;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) F[7][e] = __builtin_fmaf(s1, dprev[e], F[7][e]);
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc += F[i][e];
  sink[(int64_t)blockIdx.x * blockDim.x + t] = acc;
}

template <int KIND>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float *__restrict__ sink) {
  const int t = threadIdx.x;
  v16f acc[PROBE_CHAINS];
  v16i iacc[PROBE_CHAINS];
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c) {
    acc[c] = (v16f){};
    iacc[c] = (v16i){};
  }
  const v8i a8 = (v8i){t, 0x11111111, 0x22222222, 0x33333333, 0x04040404, 0x05050505, 0, 0};
  const v8i b8 = (v8i){0x06060606, t + 1, 0x01020304, 0x05060708, 0x0A0B0C0D, 0x01010101, 0, 0};
  const v4i a4 = (v4i){t, 0x01020304, 0x05060708, 0x0A0B0C0D};
  const v4i b4 = (v4i){0x11111111, t + 2, 0x02020202, 0x03030303};
  bf16x8 ab, bb;
  f16x8 ah, bh;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ab[k] = (__bf16)(0.25f * (k + (t & 3)));
    bb[k] = (__bf16)(0.5f * (k + 1));
    ah[k] = (_Float16)(0.25f * (k + (t & 3)));
    bh[k] = (_Float16)(0.5f * (k + 1));
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) {
#pragma unroll
      for (int c = 0; c < PROBE_CHAINS; ++c) {
        if constexpr (KIND == OQ_PROBE_FP6)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 2, 2, 0, 127, 0, 127);
        else if constexpr (KIND == OQ_PROBE_FP4)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 4, 4, 0, 127, 0, 127);
        else if constexpr (KIND == OQ_PROBE_FP8)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 0, 0, 0, 127, 0, 127);
        else if constexpr (KIND == OQ_PROBE_I8)
          iacc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, iacc[c], 0, 0, 0);
        else if constexpr (KIND == OQ_PROBE_BF16)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[c], 0, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e] + (float)iacc[c][e];
  sink[(int64_t)blockIdx.x * blockDim.x + t] = s;
}

// multiply-add pairs of one instruction (2 M N K)
double probe_ops(int kind) {
  switch (kind) {
    case OQ_PROBE_FP6:
    case OQ_PROBE_FP4:
    case OQ_PROBE_FP8: return 2.0 * 32 * 32 * 64;
    case OQ_PROBE_I8: return 2.0 * 32 * 32 * 32;
    case OQ_PROBE_FP6_UPDATE: return 2.0 * 32 * 32 * 64;
    default: return 2.0 * 32 * 32 * 16;
  }
}

}  // namespace

int probe_blocks() { return 2 * device_cus(); }

hipError_t launch_mfma_probe(int kind, int iters, float *sink, hipStream_t stream, double *ops) {
  const int blocks = probe_blocks();  // two workgroups of 4 wavefronts per CU: two wavefronts per SIMD
  if (kind == OQ_PROBE_FP6_UPDATE) {  // 8 MFMAs per wavefront per iteration
    *ops = probe_ops(kind) * (double)blocks * 4.0 * (double)iters * 8;
    hipLaunchKernelGGL(fp6_update_probe_kernel, dim3(blocks), dim3(256), 0, stream, iters, sink);
    return hipGetLastError();
  }
  *ops = probe_ops(kind) * (double)blocks * 4.0 * (double)iters * PROBE_UNROLL * PROBE_CHAINS;
  switch (kind) {
    case OQ_PROBE_FP6: hipLaunchKernelGGL(mfma_probe_kernel<OQ_PROBE_FP6>, dim3(blocks), dim3(256), 0, stream, iters, sink); break;
    case OQ_PROBE_FP4: hipLaunchKernelGGL(mfma_probe_kernel<OQ_PROBE_FP4>, dim3(blocks), dim3(256), 0, stream, iters, sink); break;
    case OQ_PROBE_FP8: hipLaunchKernelGGL(mfma_probe_kernel<OQ_PROBE_FP8>, dim3(blocks), dim3(256), 0, stream, iters, sink); break;
    case OQ_PROBE_I8: hipLaunchKernelGGL(mfma_probe_kernel<OQ_PROBE_I8>, dim3(blocks), dim3(256), 0, stream, iters, sink); break;
    case OQ_PROBE_BF16: hipLaunchKernelGGL(mfma_probe_kernel<OQ_PROBE_BF16>, dim3(blocks), dim3(256), 0, stream, iters, sink); break;
    case OQ_PROBE_F16: hipLaunchKernelGGL(mfma_probe_kernel<OQ_PROBE_F16>, dim3(blocks), dim3(256), 0, stream, iters, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oq
