// Lloyd-Max activation GEMM on the gfx950 float16 MFMA, with the weight
// prepack and the code -> level expansion that produce its operands.
//
// Arithmetic (OrbitQuant PR #25, "Default changes": Lloyd-Max activation
// codes; CentriQ Eq. 5 / Eq. 9 for the scale and rank-1 epilogue):
//   y[t][o] = bf16( rho_t * sum_k A16[t][k] W16[o][k] + m_t w1[o] + b[o] )
// A16 is the float16 level of each activation code, W16 = RN16(s q) the
// dequantized INT4 weight (code q, group scale s).  A float16 x float16
// product is exact in float32; v_mfma_f32_32x32x16_f16 sums the products in
// float32, so the only roundings are the accumulation's and the epilogue's.
//
// Tiled operand layout (rows padded to a multiple of 32, K a multiple of 16):
// chunk (r / 32, k / 16) is 1 KiB; lane l of an MFMA fragment (row l % 32,
// k 8 (l / 32) .. + 7) finds its 8 float16 at chunk + 16 l, so a fragment is
// one 16-byte LDS read per lane, conflict-free.
//
// Workgroup of 8 wavefronts, each TI x TJ MFMA tiles of 32 x 32 accumulated
// in place: TI = 4, TJ = 2 in a 2 x 4 grid (256 x 256 outputs), TI = 4,
// TJ = 3 in a 2 x 4 grid (256 x 384: a third less LDS reading per MFMA, the
// accumulators in AGPRs) or TI = 2, TJ = 3 in a 4 x 2 grid (256 x 192, for
// products whose wider tiles would leave CUs idle).  k advances in stages of
// 32 (two chunks per 32-row block): every wave copies the same share of
// each stage global -> LDS with global_load_lds_dwordx4 into a ring of
// stages (4 slots; 3 for the 384-wide tile), one barrier per stage.  A stage
// holds 8 row blocks and the tile's column blocks (a 192-wide tile loads
// two column blocks past its end and leaves them unread, so that the copies
// split evenly over the waves).
#include "oq_internal.h"

#include <cstdlib>
#include <cstring>

namespace oq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int F16_BM = 256;

// KC 16-wide chunks per stage, NSLOT stages in the LDS ring, TI x TJ tiles per wave
template <int KC, int NSLOT, int TI_ = 4, int TJ_ = 2>
struct F16C {
  static constexpr int TI = TI_, TJ = TJ_;
  static constexpr int WAVES_M = 8 / TI, WAVES_N = 8 / WAVES_M;
  static constexpr int BN = 32 * TJ * WAVES_N;
  static constexpr int SROW = 64 * TJ + 16;  // padded bytes per staged output row of 32 TJ bf16
  static constexpr int B_BLOCKS = BN == 192 ? 8 : BN / 32;
  static constexpr int A_BYTES = (F16_BM / 32) * KC * 1024;
  static constexpr int B_BYTES = B_BLOCKS * KC * 1024;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int ROWS_OFF = NSLOT * STAGE;
  static constexpr int LDS = ROWS_OFF + 2 * F16_BM * 4;
  static constexpr int PER_STAGE = (8 + B_BLOCKS) * KC / 8;  // 1 KiB copies per wave per stage
  // more than 8 tiles per wave: one register per fragment, reloaded right
  // after its last MFMA of the chunk (a second set would not fit beside
  // the accumulators)
  static constexpr bool SINGLE = TI * TJ > 8;
  static_assert(8 * PER_STAGE * 1024 == STAGE, "every wave copies the same share of a stage");
  static_assert(8 * 32 * SROW <= ROWS_OFF, "the epilogue staging fits in the ring");
  static_assert(32 * TI * WAVES_M == F16_BM && BN <= 384, "workgroup shape");
  static_assert(LDS <= 160 * 1024, "LDS");
  // chunk 0 of stage g + 1 is read during stage g, so stage g + 1 must be in
  // flight before stage g starts (NSLOT >= 3); the waits below count exactly
  // for three or four slots
  static_assert(NSLOT == 3 || NSLOT == 4, "ring depth");
  static_assert(PER_STAGE * (NSLOT - 2) <= 63, "vmcnt range");
};

template <int C>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (C & 0xF) | ((C >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int KC, int NSLOT, int TI, int TJ>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_f16_kernel(const uint8_t *__restrict__ A, const float *__restrict__ a_scale, int64_t M, int K,
                const uint8_t *__restrict__ W, int N, int Np, const float *__restrict__ mean,
                const float *__restrict__ w1, const float *__restrict__ bias, uint16_t *__restrict__ y, int64_t ldy) {
  using C = F16C<KC, NSLOT, TI, TJ>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t lds0 = lds_addr_of(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KCH = K / 16;
  const int S = KCH / KC;
  const int64_t m0 = (int64_t)blockIdx.y * F16_BM;
  const int n0 = blockIdx.x * C::BN;
  const int64_t mblocks = (M + 31) / 32;
  const int nblocks = Np / 32;

  // copy units of this wave: u = wave + 8 q; units 0 .. 8 KC - 1 are A chunks
  // (row block u / KC, chunk u % KC of the stage), the rest the same for W;
  // unit u lands at 1 KiB * u of the slot.  Blocks past the operand end
  // re-read the last block (their outputs are never stored).
  const uint8_t *cptr[C::PER_STAGE];
  uint32_t clds[C::PER_STAGE];
#pragma unroll
  for (int q = 0; q < C::PER_STAGE; ++q) {
    const int u = wave + 8 * q;
    if (u < 8 * KC) {
      int64_t rb = m0 / 32 + u / KC;
      if (rb > mblocks - 1) rb = mblocks - 1;
      cptr[q] = A + (rb * KCH + u % KC) * 1024 + 16 * lane;
    } else {
      const int uu = u - 8 * KC;
      int cb = n0 / 32 + uu / KC;
      if (cb > nblocks - 1) cb = nblocks - 1;
      cptr[q] = W + ((int64_t)cb * KCH + uu % KC) * 1024 + 16 * lane;
    }
    clds[q] = 1024u * u;
  }
  auto issue = [&](int slot, int st) {
    const uint32_t base = lds0 + slot * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::PER_STAGE; ++q) dma_lds16(cptr[q] + (int64_t)st * (KC * 1024), base + clds[q]);
  };

  float *lds_alpha = reinterpret_cast<float *>(smem + C::ROWS_OFF);
  float *lds_mean = lds_alpha + F16_BM;
  for (int t = threadIdx.x; t < F16_BM; t += 512) {
    const int64_t row = m0 + t;
    lds_alpha[t] = row < M ? a_scale[row] : 0.f;
    lds_mean[t] = (mean && row < M) ? mean[row] : 0.f;
  }

  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int r = lane & 31, half = lane >> 5;
  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = (v16f){};

  // A fragment (row block wm * TI + i, chunk kc) and B fragment (column block
  // wn * TJ + j, chunk kc) of the stage in slot `slot`
  const uint8_t *fa = smem + 16 * lane + (wm * TI) * KC * 1024;
  const uint8_t *fb = smem + 16 * lane + C::A_BYTES + (wn * TJ) * KC * 1024;
  auto load = [&](v8h (&a)[TI], v8h (&b)[TJ], int slot, int kc) {
#pragma unroll
    for (int i = 0; i < TI; ++i) a[i] = *reinterpret_cast<const v8h *>(fa + slot * C::STAGE + (i * KC + kc) * 1024);
#pragma unroll
    for (int j = 0; j < TJ; ++j) b[j] = *reinterpret_cast<const v8h *>(fb + slot * C::STAGE + (j * KC + kc) * 1024);
  };
  auto mma = [&](const v8h (&a)[TI], const v8h (&b)[TJ]) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
  };

  // Schedule: each stage starts with its first chunk's fragments in registers.
  // Stage g: wait for this wave's copies of stage g + 1 and for its LDS
  // reads, barrier (stage g + 1 is then visible everywhere and nobody reads
  // the slot of stage g - 1 any more), refill that slot with stage
  // g + NSLOT - 1; the fragments of the next chunk (of this stage, or chunk 0
  // of stage g + 1) are read under the MFMAs of the current one.
#pragma unroll
  for (int p = 0; p < NSLOT - 1; ++p)
    if (p < S) issue(p, p);
  // stage 0 is complete once at most the later prologue stages are outstanding
  if constexpr (NSLOT >= 4) {
    if (S > 2) wait_vm<2 * C::PER_STAGE>();
    else if (S > 1) wait_vm<C::PER_STAGE>();
    else wait_vm<0>();
  } else {
    if (S > 1) wait_vm<C::PER_STAGE>();
    else wait_vm<0>();
  }
  __builtin_amdgcn_s_barrier();
  if constexpr (C::SINGLE) {
    // tiles column-major (i fastest), so a[i] is reloaded after tile
    // (i, TJ - 1) and b[j] after tile (TI - 1, j), each at least TI tiles
    // before its next use
    v8h a[TI], b[TJ];
    load(a, b, 0, 0);
    for (int g = 0; g < S; ++g) {
      if constexpr (NSLOT >= 4) {
        if (g + 2 < S) wait_vm<(NSLOT - 3) * C::PER_STAGE>();
        else wait_vm<0>();
      } else {
        wait_vm<0>();
      }
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      if (g + NSLOT - 1 < S) issue((g + NSLOT - 1) % NSLOT, g + NSLOT - 1);
      __builtin_amdgcn_sched_barrier(0);
      const int slot = g % NSLOT;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        // the next chunk: this stage's next, or chunk 0 of the next stage
        // (after the last stage a slot whose contents are never used)
        const int ns = kc + 1 < KC ? slot : (g + 1) % NSLOT, nk = kc + 1 < KC ? kc + 1 : 0;
#pragma unroll
        for (int t = 0; t < TI * TJ; ++t) {
          const int i = t % TI, j = t / TI;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
          if (j == TJ - 1) a[i] = *reinterpret_cast<const v8h *>(fa + ns * C::STAGE + (i * KC + nk) * 1024);
          if (i == TI - 1) b[j] = *reinterpret_cast<const v8h *>(fb + ns * C::STAGE + (j * KC + nk) * 1024);
        }
      }
    }
  } else {
  v8h fr[2][TI], gr[2][TJ];
  load(fr[0], gr[0], 0, 0);

  for (int g = 0; g < S; ++g) {
    // stages issued after g + 1 so far: g + 2 .. g + NSLOT - 2
    if constexpr (NSLOT >= 4) {
      if (g + 2 < S) wait_vm<(NSLOT - 3) * C::PER_STAGE>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if (g + NSLOT - 1 < S) issue((g + NSLOT - 1) % NSLOT, g + NSLOT - 1);
    __builtin_amdgcn_sched_barrier(0);
    const int slot = g % NSLOT;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      // after the last stage the final read targets a slot whose contents are never used
      if (kc + 1 < KC) load(fr[(kc + 1) & 1], gr[(kc + 1) & 1], slot, kc + 1);
      else load(fr[(kc + 1) & 1], gr[(kc + 1) & 1], (g + 1) % NSLOT, 0);
      mma(fr[kc & 1], gr[kc & 1]);
    }
    if constexpr (KC & 1) {  // the next stage starts from buffer 0
#pragma unroll
      for (int i = 0; i < TI; ++i) fr[0][i] = fr[1][i];
#pragma unroll
      for (int j = 0; j < TJ; ++j) gr[0][j] = gr[1][j];
    }
  }

  }

  // ---- epilogue: y = rho F + m w1 + b, bf16, staged per 32-row slab in this
  // wave's own LDS area (the ring is free once every wave has passed the
  // barrier) so that the global writes are 16-byte runs
  __syncthreads();
  constexpr int SROW = C::SROW;
  float w1v[TJ], bv[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int col = n0 + wn * 32 * TJ + 32 * j + r;
    w1v[j] = bv[j] = 0.f;
    if (col < N) {
      if (mean) w1v[j] = w1[col];
      if (bias) bv[j] = bias[col];
    }
  }
  uint8_t *stg = smem + wave * (32 * SROW);
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(y) & 15) == 0) && (ldy % 8 == 0);
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      // rows e4 * 8 + half * 4 + 0..3 of this 32-row slab
      const int rl = wm * 32 * TI + 32 * i + e4 * 8 + half * 4;
      const float4 al4 = *reinterpret_cast<const float4 *>(lds_alpha + rl);
      const float4 mu4 = *reinterpret_cast<const float4 *>(lds_mean + rl);
      const float al[4] = {al4.x, al4.y, al4.z, al4.w}, mu[4] = {mu4.x, mu4.y, mu4.z, mu4.w};
#pragma unroll
      for (int e1 = 0; e1 < 4; ++e1) {
        const int e = 4 * e4 + e1;
        const int rr = e4 * 8 + half * 4 + e1;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          float v = al[e1] * acc[i][j][e];
          if (mean) v = __builtin_fmaf(mu[e1], w1v[j], v);
          if (bias) v = v + bv[j];
          *reinterpret_cast<uint16_t *>(stg + rr * SROW + (32 * j + r) * 2) = f32_to_bf16_rne(v);
        }
      }
    }
    // the slab is 32 rows of 4 TJ 16-byte pieces: 2 TJ rounds of 64 pieces
    constexpr int CPR = 4 * TJ;
#pragma unroll
    for (int q = 0; q < 2 * TJ; ++q) {
      const int piece = lane + 64 * q;
      const int rr = piece / CPR, cl = (piece % CPR) * 8;
      const int col = n0 + wn * 32 * TJ + cl;
      const int64_t row = m0 + wm * 32 * TI + 32 * i + rr;
      const uint4 v = *reinterpret_cast<const uint4 *>(stg + rr * SROW + cl * 2);
      if (row >= M) continue;
      uint16_t *dst = y + row * ldy + col;
      if (vec_ok && col + 8 <= N) {
        *reinterpret_cast<uint4 *>(dst) = v;
      } else {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (col + c < N) dst[c] = (uint16_t)(wv[c >> 1] >> (16 * (c & 1)));
      }
    }
  }
}

// RN16(s * q) for an INT4 code q: the float32 product is made round-to-odd
// (truncated toward zero, last bit set when inexact, the error coming exact
// from an fma), and float32 has 13 bits more than float16, so rounding that
// to float16 rounds the exact product once.
__device__ __forceinline__ uint32_t rn16_scaled(float s, int q) {
  const float fq = (float)q;
  const float p = s * fq;
  const float e = __builtin_fmaf(s, fq, -p);
  uint32_t b = __float_as_uint(p);
  if (e != 0.f) {
    if ((e < 0.f) != (p < 0.f)) b -= 1u;  // |s q| < |p|: step toward zero
    b |= 1u;
  }
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(b));
}

// canonical INT4 nibbles + scales [N][K / group] -> W16 tiled [Np / 32][K / 16][1 KiB]
// one thread per 16-byte lane piece; consecutive threads write consecutive pieces
__global__ void prepack_w16_kernel(const uint8_t *__restrict__ w, const float *__restrict__ ws, int N, int Np, int K,
                                   int group, uint8_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KCH = K / 16;
  const int64_t total = (int64_t)(Np / 32) * KCH * 64;
  if (idx >= total) return;
  const int l = (int)(idx & 63);
  const int64_t cc = idx >> 6;
  const int ch = (int)(cc % KCH);
  const int64_t cb = cc / KCH;
  const int64_t o = cb * 32 + (l & 31);
  const int k0 = ch * 16 + 8 * (l >> 5);
  uint32_t hv[4] = {0u, 0u, 0u, 0u};
  if (o < N) {
    const uint32_t nib = *reinterpret_cast<const uint32_t *>(w + o * (K / 2) + k0 / 2);
    const float s = ws[o * (K / group) + k0 / group];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int q = (int)((nib >> (4 * j)) & 0xF);
      q = q >= 8 ? q - 16 : q;
      hv[j >> 1] |= rn16_scaled(s, q) << (16 * (j & 1));
    }
  }
  *reinterpret_cast<uint4 *>(out + idx * 16) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
}

// canonical Lloyd-Max codes (nibbles or bytes, [M][ldc]) -> tiled float16
// levels [Mp / 32][K / 16][1 KiB]; padding rows get zeros
__global__ void lm_expand_kernel(const uint8_t *__restrict__ codes, int64_t ldc, int nibbles,
                                 const uint16_t *__restrict__ levels, int nlev, int64_t M, int K,
                                 uint8_t *__restrict__ out) {
  __shared__ uint16_t lv[256];
  for (int t = threadIdx.x; t < 256; t += blockDim.x) lv[t] = t < nlev ? levels[t] : (uint16_t)0;
  __syncthreads();
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KCH = K / 16;
  const int64_t total = (M + 31) / 32 * KCH * 64;
  if (idx >= total) return;
  const int l = (int)(idx & 63);
  const int64_t cc = idx >> 6;
  const int ch = (int)(cc % KCH);
  const int64_t row = (cc / KCH) * 32 + (l & 31);
  const int k0 = ch * 16 + 8 * (l >> 5);
  uint32_t hv[4] = {0u, 0u, 0u, 0u};
  if (row < M) {
    uint32_t c[8];
    if (nibbles) {
      const uint32_t wd = *reinterpret_cast<const uint32_t *>(codes + row * ldc + k0 / 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = (wd >> (4 * j)) & 0xFu;
    } else {
      const uint2 wd = *reinterpret_cast<const uint2 *>(codes + row * ldc + k0);
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = ((j < 4 ? wd.x : wd.y) >> (8 * (j & 3))) & 0xFFu;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) hv[j >> 1] |= (uint32_t)lv[c[j]] << (16 * (j & 1));
  }
  *reinterpret_cast<uint4 *>(out + idx * 16) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
}

template <int KC, int NSLOT, int TI, int TJ>
hipError_t launch_f16(const uint8_t *A, const float *a_scale, int64_t M, int K, const uint8_t *W, int N, int Np,
                      const float *mean, const float *w1, const float *bias, uint16_t *y, int64_t ldy,
                      hipStream_t stream) {
  using C = F16C<KC, NSLOT, TI, TJ>;
  static std::atomic<bool> attr_set[64];
  const hipError_t e = lds_limit_once((const void *)gemm_f16_kernel<KC, NSLOT, TI, TJ>, C::LDS, attr_set);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((N + C::BN - 1) / C::BN), (unsigned)((M + F16_BM - 1) / F16_BM));
  hipLaunchKernelGGL((gemm_f16_kernel<KC, NSLOT, TI, TJ>), grid, dim3(512), C::LDS, stream, A, a_scale, M, K, W, N, Np,
                     mean, w1, bias, y, ldy);
  return hipGetLastError();
}

// Tile width: the one whose whole waves of workgroups (one per CU) cover the
// fewest output columns, the wider on a tie (4096 x 3072 on 256 CUs: 256
// tiles of 256 x 192; 4096 x 12288: 512 tiles of 256 x 384).
// OQ_F16_TILE=256x384, 256x256 or 256x192 in the environment forces one
// (for tuning and tests).
int f16_width(int64_t M, int N) {
  if (const char *f = getenv("OQ_F16_TILE")) {
    if (strcmp(f, "256x384") == 0) return 384;
    if (strcmp(f, "256x256") == 0) return 256;
    if (strcmp(f, "256x192") == 0) return 192;
  }
  const int64_t cus = device_cus();
  const int64_t mt = (M + 255) / 256;
  auto covered = [&](int w) { return (mt * ((N + w - 1) / w) + cus - 1) / cus * w; };
  const int64_t c384 = covered(384), c256 = covered(256), c192 = covered(192);
  if (c384 <= c256 && c384 <= c192) return 384;
  return c256 <= c192 ? 256 : 192;
}

}  // namespace

hipError_t launch_gemm_f16(const uint8_t *A, const float *a_scale, int64_t M, int K, const uint8_t *W, int N,
                           const float *mean, const float *w1, const float *bias, uint16_t *y, int64_t ldy,
                           hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int Np = (N + 31) / 32 * 32;
  const int w = f16_width(M, N);
  if (w == 192) return launch_f16<2, 4, 2, 3>(A, a_scale, M, K, W, N, Np, mean, w1, bias, y, ldy, stream);
  if (w == 384) return launch_f16<2, 3, 4, 3>(A, a_scale, M, K, W, N, Np, mean, w1, bias, y, ldy, stream);
  return launch_f16<2, 4, 4, 2>(A, a_scale, M, K, W, N, Np, mean, w1, bias, y, ldy, stream);
}

hipError_t launch_prepack_w16(const uint8_t *w, const float *ws, int N, int K, int group, uint8_t *out,
                              hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int Np = (N + 31) / 32 * 32;
  const int64_t total = (int64_t)(Np / 32) * (K / 16) * 64;
  hipLaunchKernelGGL(prepack_w16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, w, ws, N, Np, K,
                     group, out);
  return hipGetLastError();
}

hipError_t launch_lm_expand(const uint8_t *codes, int64_t ldc, int nibbles, const uint16_t *levels, int nlev,
                            int64_t M, int K, uint8_t *out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t total = (M + 31) / 32 * (K / 16) * 64;
  hipLaunchKernelGGL(lm_expand_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, codes, ldc,
                     nibbles, levels, nlev, M, K, out);
  return hipGetLastError();
}

}  // namespace oq
