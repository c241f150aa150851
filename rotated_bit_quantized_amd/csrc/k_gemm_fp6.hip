// Tiled W4A4 / W4A6 GEMM on the gfx950 scaled FP6 MFMA, plus the weight
// prepack kernel that produces its operand layout.
//
// Arithmetic (CentriQ Eq. 5 / Eq. 9 with the per-(row, group) weight scale of
// Sec. 3 Eq. 2):  y = bf16( a_scale[t] * sum_g s[o,g] acc_g[t,o] + m_t w1[o] + b[o] ).
//
// Integer codes in [-7, 7] are exact FP6 E2M3 values, so with unit E8M0
// scales v_mfma_scale_f32_32x32x64_f8f6f4 returns the exact group sum
// acc_g (|acc_g| <= 64*7*7 < 2^24) as a float32.  6-bit activation codes
// q in [-31, 31] are split as q = 8 qh + ql with qh in [-4, 3] and ql in
// [0, 7] (two planes); the high plane runs with an E8M0 scale of 2^3 and the
// low plane accumulates onto it, again exactly.  The fp32 update per group is
// the same fma(s, acc, F) as the int8-MFMA kernel, so both kernels produce
// bit-identical outputs.
//
// Tiled operand layout (rows padded to a multiple of 32, K a multiple of 64):
//   row r, k-group kg = k / 64 occupies 48 bytes split into six 8-byte chunks;
//   chunk c of (r, kg) is at ((r/32) * (K/64) + kg) * 1536 + c * 256 + (r%32) * 8
//   and holds bits [64c, 64c + 64) of the 384-bit string in which value
//   j = k % 64 occupies bits [6j, 6j + 6).  Lane l of an MFMA fragment (row
//   l % 32, k-half l / 32) reads chunks 3(l/32) .. 3(l/32)+2: 24 bytes = its
//   32 FP6 values, and the 32 lanes of a half read 256 contiguous bytes.
// Weight scales are stored transposed, [K/64][N_padded] float32.
//
// Workgroup: WM x WN wavefronts, each computing 128 x 64 outputs (4 x 2 MFMA
// tiles of 32 x 32).  The k loop walks the 64-wide groups; each group's A, B
// and scale tiles are copied global -> LDS with global_load_lds_dwordx4
// (no register staging) into a 3-stage ring, one barrier per group.
#include "oq_internal.h"

namespace oq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int CHUNK_TILE = 1536;  // bytes of one 32-row x 64-k tile
constexpr int STAGES = 3;

__device__ __forceinline__ void dma16(const void *g, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ v8i frag(const uint8_t *tile, int half, int r) {
  const uint8_t *p = tile + (3 * half) * 256 + r * 8;
  const uint2 a = *reinterpret_cast<const uint2 *>(p);
  const uint2 b = *reinterpret_cast<const uint2 *>(p + 256);
  const uint2 c = *reinterpret_cast<const uint2 *>(p + 512);
  return (v8i){(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
}

template <int WM, int WN, int PLANES>
struct Cfg {
  static constexpr int BM = 128 * WM, BN = 64 * WN;
  static constexpr int A_BYTES = PLANES * (BM / 32) * CHUNK_TILE;
  static constexpr int B_BYTES = (BN / 32) * CHUNK_TILE;
  static constexpr int S_BYTES = 1024;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int UNITS = STAGE / 1024;          // 1 KiB DMA units per stage
  static constexpr int WAVES = WM * WN;
  static constexpr int UPW = (UNITS + WAVES - 1) / WAVES;
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "stage regions must be whole units");
};

template <int WM, int WN, int PLANES>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_fp6_kernel(const uint8_t *__restrict__ A, int64_t a_plane_bytes, const float *__restrict__ a_scale, int64_t M,
                int K, const uint8_t *__restrict__ W, const float *__restrict__ wst, int N, int Np,
                const float *__restrict__ mean, const float *__restrict__ w1, const float *__restrict__ bias,
                uint16_t *__restrict__ y, int64_t ldy) {
  using C = Cfg<WM, WN, PLANES>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = K / 64;
  const int64_t m0 = (int64_t)blockIdx.y * C::BM;
  const int n0 = blockIdx.x * C::BN;
  const int64_t mblocks = (M + 31) / 32;
  const int nblocks = Np / 32;

  // ---- per-lane DMA sources for the units this wave copies (k-group 0)
  const uint8_t *src[C::UPW];
  int64_t inc[C::UPW];
  int uoff[C::UPW];
#pragma unroll
  for (int q = 0; q < C::UPW; ++q) {
    const int u = wave + q * C::WAVES;
    uoff[q] = u < C::UNITS ? u * 1024 : -1;
    const int o = (u < C::UNITS ? u : 0) * 1024 + lane * 16;
    if (o < C::A_BYTES) {
      const int p = o / ((C::BM / 32) * CHUNK_TILE);
      const int oo = o % ((C::BM / 32) * CHUNK_TILE);
      int64_t rb = m0 / 32 + oo / CHUNK_TILE;
      if (rb >= mblocks) rb = mblocks - 1;
      src[q] = A + p * a_plane_bytes + rb * G * CHUNK_TILE + oo % CHUNK_TILE;
      inc[q] = CHUNK_TILE;
    } else if (o < C::A_BYTES + C::B_BYTES) {
      const int oo = o - C::A_BYTES;
      int cb = n0 / 32 + oo / CHUNK_TILE;
      if (cb >= nblocks) cb = nblocks - 1;
      src[q] = W + (int64_t)cb * G * CHUNK_TILE + oo % CHUNK_TILE;
      inc[q] = CHUNK_TILE;
    } else {
      int c = n0 + (o - C::A_BYTES - C::B_BYTES) / 4;
      if (c > Np - 4) c = Np - 4;
      src[q] = reinterpret_cast<const uint8_t *>(wst + c);
      inc[q] = (int64_t)Np * 4;
    }
  }

  auto issue = [&](int ks) {
    uint8_t *stage = smem + (ks % STAGES) * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::UPW; ++q)
      if (uoff[q] >= 0) dma16(src[q] + (int64_t)ks * inc[q], stage + uoff[q]);
  };

  const int nq = (C::UNITS - wave + C::WAVES - 1) / C::WAVES;  // units this wave copies per group
  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, half = lane >> 5;

  float F[4][2][16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) F[i][j][e] = 0.f;

  issue(0);
  if (G > 1) issue(1);
  for (int ks = 0; ks < G; ++ks) {
    // wait until this wave's copies for group ks have landed: the copies of
    // group ks+1 (nq per wave) may still be in flight
    if (ks + 1 < G) {
      if (nq == C::UPW)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (C::UPW & 0xF));
      else
        __builtin_amdgcn_s_waitcnt(0x0F70 | ((C::UPW - 1) & 0xF));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    // a bare barrier: the wait above already covers this wave's copies, and a
    // fenced __syncthreads() would also drain the copies of group ks+1
    __builtin_amdgcn_s_barrier();
    if (ks + 2 < G) issue(ks + 2);

    const uint8_t *stage = smem + (ks % STAGES) * C::STAGE;
    const uint8_t *sA = stage;
    const uint8_t *sB = stage + C::A_BYTES;
    const float *sS = reinterpret_cast<const float *>(stage + C::A_BYTES + C::B_BYTES);
    v8i b[2];
    float s[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      b[j] = frag(sB + (wn * 2 + j) * CHUNK_TILE, half, r);
      s[j] = sS[wn * 64 + 32 * j + r];
    }
    // software pipeline over the 8 tiles: the MFMA of tile t+1 is issued
    // before the fp32 updates of tile t, so the matrix core and the VALU overlap
    v16f dprev = (v16f){};
#pragma unroll
    for (int t = 0; t <= 8; ++t) {
      v16f dnext;
      if (t < 8) {
        const int i = t >> 1, j = t & 1;
        const v8i a = frag(sA + (wm * 4 + i) * CHUNK_TILE, half, r);
        if (PLANES == 2) {
          const v8i a2 = frag(sA + (C::BM / 32) * CHUNK_TILE + (wm * 4 + i) * CHUNK_TILE, half, r);
          dnext = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[j], (v16f){}, 2, 2, 0, 130, 0, 127);
          dnext = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a2, b[j], dnext, 2, 2, 0, 127, 0, 127);
        } else {
          dnext = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[j], (v16f){}, 2, 2, 0, 127, 0, 127);
        }
      }
      if (t > 0) {
        const int i = (t - 1) >> 1, j = (t - 1) & 1;
#pragma unroll
        for (int e = 0; e < 16; ++e) F[i][j][e] = __builtin_fmaf(s[j], dprev[e], F[i][j][e]);
      }
      if (t < 8) dprev = dnext;
    }
  }

  // ---- epilogue: y = a_scale * F + mean * w1 + bias (same order as the int8 kernel)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = m0 + wm * 128 + 32 * i + (e >> 2) * 8 + half * 4 + (e & 3);
      if (row >= M) continue;
      const float al = a_scale[row];
      const float mu = mean ? mean[row] : 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + 32 * j + r;
        if (col >= N) continue;
        float v = al * F[i][j][e];
        if (mean) v = __builtin_fmaf(mu, w1[col], v);
        if (bias) v = v + bias[col];
        y[row * ldy + col] = f32_to_bf16_rne(v);
      }
    }
  }
}

// canonical INT4 nibbles + scales [N][G] -> tiled FP6 [Np/32][G][1536] + scales [G][Np]
__global__ void prepack_w4_kernel(const uint8_t *__restrict__ w, const float *__restrict__ ws, int N, int Np, int K,
                                  uint8_t *__restrict__ out, float *__restrict__ out_s) {
  // one thread per (row, k-group, half): 32 codes -> 24 bytes
  const int G = K / 64;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)Np * G * 2;
  if (idx >= total) return;
  const int half = (int)(idx & 1);
  const int64_t rg = idx >> 1;
  const int kg = (int)(rg % G);
  const int row = (int)(rg / G);
  uint32_t c[32];
  if (row < N) {
    const uint4 p = *reinterpret_cast<const uint4 *>(w + (int64_t)row * (K / 2) + kg * 32 + half * 16);
    const uint32_t wd[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      int q = (int)((wd[j >> 3] >> (4 * (j & 7))) & 0xF);
      q = q >= 8 ? q - 16 : q;
      c[j] = fp6_e2m3_of_int(q);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = 0;
  }
  uint32_t bits[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int b = 6 * j;
    bits[b >> 5] |= c[j] << (b & 31);
    if ((b & 31) > 26) bits[(b >> 5) + 1] |= c[j] >> (32 - (b & 31));
  }
  uint8_t *tile = out + ((int64_t)(row / 32) * G + kg) * CHUNK_TILE + (row % 32) * 8;
#pragma unroll
  for (int q = 0; q < 3; ++q)
    *reinterpret_cast<uint2 *>(tile + (3 * half + q) * 256) = make_uint2(bits[2 * q], bits[2 * q + 1]);
  if (half == 0) out_s[(int64_t)kg * Np + row] = row < N ? ws[(int64_t)row * G + kg] : 0.f;
}

template <int WM, int WN, int PLANES>
hipError_t launch_cfg(const uint8_t *A, int64_t a_plane_bytes, const float *a_scale, int64_t M, int K,
                      const uint8_t *W, const float *wst, int N, int Np, const float *mean, const float *w1,
                      const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream) {
  using C = Cfg<WM, WN, PLANES>;
  const size_t lds = (size_t)STAGES * C::STAGE;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)gemm_fp6_kernel<WM, WN, PLANES>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)((N + C::BN - 1) / C::BN), (unsigned)((M + C::BM - 1) / C::BM));
  hipLaunchKernelGGL((gemm_fp6_kernel<WM, WN, PLANES>), grid, dim3(64 * C::WAVES), lds, stream, A, a_plane_bytes,
                     a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp6(const uint8_t *A, int planes, const float *a_scale, int64_t M, int K, const uint8_t *W,
                           const float *wst, int N, const float *mean, const float *w1, const float *bias,
                           uint16_t *y, int64_t ldy, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int Np = (N + 31) / 32 * 32;
  const int64_t plane = tiled_bytes(M, K);
  if (planes == 2) return launch_cfg<2, 4, 2>(A, plane, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy, stream);
  return launch_cfg<2, 4, 1>(A, plane, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy, stream);
}

hipError_t launch_prepack_w4(const uint8_t *w, const float *ws, int N, int K, uint8_t *out, float *out_s,
                             hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int Np = (N + 31) / 32 * 32;
  const int64_t total = (int64_t)Np * (K / 64) * 2;
  hipLaunchKernelGGL(prepack_w4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, w, ws, N, Np, K,
                     out, out_s);
  return hipGetLastError();
}

}  // namespace oq
