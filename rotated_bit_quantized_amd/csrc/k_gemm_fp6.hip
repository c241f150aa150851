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
//   tile (r/32, kg = k / 64) is 1536 contiguous bytes.  Lane l of an MFMA
//   fragment (row l % 32, k-half l / 32) needs the 32 FP6 values of its row and
//   half as a 192-bit string (value j in bits [6j, 6j + 6)); its bytes 0..15
//   sit at tile + 16 l and bytes 16..23 at tile + 1024 + 8 l, so a fragment is
//   one 16-byte and one 8-byte LDS read per lane, both conflict-free.
// Weight scales are stored transposed, [K/64][N_padded] float32.
//
// Asymmetric weights (CentriQ Sec. 3 Eq. 2, stored as Q - 8 per App. B.2):
// the codes q' = Q - 8 lie in [-8, 7]; -8 is no FP6 E2M3 value, but q'/2 is
// (every half-integer in [-4, 3.5]), so the prepack stores q'/2 and the MFMA
// takes an E8M0 scale of 2^1 for the weights: the group sums stay exact.  The
// real shift leaves -sum_g C_g p_g (C = sigma (z - 8) per row and group, p the
// group sums of the activation codes), a product of depth K/64 computed once
// per tile after the main loop on bfloat16 matrix cores, with p and C split
// into pieces that make every product exact in float32.
//
// The kernel walks the 64-wide k groups; each group's A, B and scale tiles
// are copied global -> LDS with global_load_lds (no register staging) into a
// ring of stages.  Single-plane (4-bit) and two-plane (6-bit) activations run
// the same kernel; its shapes and schedule are described at its definition.
#include "oq_internal.h"

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#ifndef FP6_SLOTS
#define FP6_SLOTS 4
#endif
#ifndef FP6_PAIRED
#define FP6_PAIRED true
#endif

namespace oq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int CHUNK_TILE = 1536;  // bytes of one 32-row x 64-k tile


// MFMA operand of lane l (row l % 32, k-half l / 32) from one tile: its 24
// bytes are at tile + 16 l (16 bytes) and tile + 1024 + 8 l (8 bytes)
__device__ __forceinline__ v8i frag_at(const uint8_t *main16, const uint8_t *tail8) {
  const uint4 a = *reinterpret_cast<const uint4 *>(main16);
  const uint2 b = *reinterpret_cast<const uint2 *>(tail8);
  return (v8i){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, 0, 0};
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
  uint8_t *tile = out + ((int64_t)(row / 32) * G + kg) * CHUNK_TILE;
  const int l = 32 * half + row % 32;
  *reinterpret_cast<uint4 *>(tile + 16 * l) = make_uint4(bits[0], bits[1], bits[2], bits[3]);
  *reinterpret_cast<uint2 *>(tile + 1024 + 8 * l) = make_uint2(bits[4], bits[5]);
  if (half == 0) out_s[(int64_t)kg * Np + row] = row < N ? ws[(int64_t)row * G + kg] : 0.f;
}

// FP6 E2M3 bits of q'/2 for an asymmetric code q' in [-8, 7]: |q'|/2 in
// {0, 0.5, .., 4} -> 0x00 0x04 0x08 0x0C 0x10 0x12 0x14 0x16 0x18, sign bit 5
__device__ __forceinline__ uint32_t fp6_e2m3_of_half(int q) {
  const uint32_t a = (uint32_t)(q < 0 ? -q : q);
  const uint32_t code = a == 8 ? 0x18u : (__builtin_amdgcn_perm(0x16141210u, 0x0C080400u, a) & 0xFFu);
  return code | (q < 0 ? 0x20u : 0u);
}

// canonical asymmetric codes q' = Q - 8 [N][K/2] + bfloat16 sigma, z [N][G] ->
// tiled FP6 of q'/2, sigma transposed [G][Np] float32, and C = RN32(sigma
// RN32(z - 8)) transposed [G][Np] as the three bfloat16 pieces of -C (the
// truncation split C = c1 + c2 + c3, each exactly a bfloat16), packed as
// (-c1 | -c2 << 16, -c3) (padding rows: zero codes, scale and C)
__global__ void prepack_w4a_kernel(const uint8_t *__restrict__ w, const uint16_t *__restrict__ sig,
                                   const uint16_t *__restrict__ zero, int N, int Np, int K, uint8_t *__restrict__ out,
                                   float *__restrict__ out_s, uint2 *__restrict__ out_c) {
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
      c[j] = fp6_e2m3_of_half(q);
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
  uint8_t *tile = out + ((int64_t)(row / 32) * G + kg) * CHUNK_TILE;
  const int l = 32 * half + row % 32;
  *reinterpret_cast<uint4 *>(tile + 16 * l) = make_uint4(bits[0], bits[1], bits[2], bits[3]);
  *reinterpret_cast<uint2 *>(tile + 1024 + 8 * l) = make_uint2(bits[4], bits[5]);
  if (half == 0) {
    float sv = 0.f, cv = 0.f;
    if (row < N) {
      sv = __uint_as_float((uint32_t)sig[(int64_t)row * G + kg] << 16);
      const float zv = __uint_as_float((uint32_t)zero[(int64_t)row * G + kg] << 16);
      cv = sv * (zv - 8.0f);
    }
    const uint32_t c1 = __float_as_uint(cv) & 0xFFFF0000u;
    const float rem = cv - __uint_as_float(c1);
    const uint32_t c2 = __float_as_uint(rem) & 0xFFFF0000u;
    const uint32_t c3 = __float_as_uint(rem - __uint_as_float(c2));
    const uint32_t n1 = (c1 ^ 0x80000000u) >> 16, n2 = (c2 ^ 0x80000000u) >> 16, n3 = (c3 ^ 0x80000000u) >> 16;
    out_s[(int64_t)kg * Np + row] = sv;
    out_c[(int64_t)kg * Np + row] = make_uint2(n1 | (n2 << 16), n3);
  }
}

// ---------------------------------------------------------------------------
// Single-plane kernel with the fragments of the next k-group prefetched into
// registers while the current group computes.  Workgroups of 8 or 4 waves
// (shapes below), a 4-slot ring of one k-group per slot and one barrier per
// two groups:
//   before groups g, g+1: own copies of stages g+1, g+2 done (vmcnt) and own
//   LDS reads done (lgkmcnt) -> barrier -> refill the two slots read during
//   the previous two groups with stages g+3, g+4;
//   during group g: each fragment of g+1 is loaded into its register right
//   after the last MFMA of g that reads it, the scales of g+1 at the start.
//   So every group starts with its operands in registers.
// Copies use an SGPR base per unit plus a loop-invariant per-lane offset.
// The loop is unrolled by the ring depth, so LDS addresses are immediates.
// ---------------------------------------------------------------------------
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int C>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (C & 0xF) | ((C >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup shapes: each wave computes TI x TJ MFMA tiles of 32 x 32.
//   8 waves, TI = 4, TJ = 2: waves 2 (rows) x 4 (columns), 256 x 256 outputs;
//   8 waves, TI = 2, TJ = 3: waves 4 x 2, 256 x 192 outputs;
//   8 waves, TI = 2, TJ = 2: waves 4 x 2, 256 x 128 outputs;
//   4 waves, TI = 4, TJ = 2: waves 2 x 2, 256 x 128 outputs;
//   4 waves, TI = 2, TJ = 3: waves 2 x 2, 128 x 192 outputs.
// An 8-wave stage holds 8 A tiles per plane and 256 scales whatever the
// shape, and exactly its B tiles where that splits the copies evenly over
// the waves (256 and 128 wide); a 192-wide tile loads the two column blocks
// past its end too and leaves them unread.  A 4-wave stage holds exactly its
// tiles.  The code bytes of a
// stage are split evenly over the waves as U4 1 KiB units (16 bytes a lane)
// and U1 256-byte units (4 bytes a lane), and every wave copies one 256-byte
// chunk of scales, so all waves issue the same copies per stage and the
// vmcnt values are compile-time constants.  (The paired schedule of 8-wave
// workgroups hands the units of waves w + 4 to waves w and copies each scale
// chunk once; it waits for all copies before each barrier.)  4-wave workgroups fit two to a CU
// (LDS under 80 KiB, the epilogue staging reusing the ring), so one
// workgroup's barrier waits and epilogue overlap the other's main loop.
template <int NSLOT_, int TI_, int TJ_, int WAVES_, int PLANES_>
struct V2C {
  static constexpr int WAVES = WAVES_, TI = TI_, TJ = TJ_, NSLOT = NSLOT_, PLANES = PLANES_;
  static constexpr int WAVES_M = WAVES == 8 ? 8 / TI : 2, WAVES_N = WAVES / WAVES_M;
  static constexpr int BM = 32 * TI * WAVES_M, BN = 32 * TJ * WAVES_N;
  static constexpr int A_BYTES = (WAVES == 8 ? 8 : BM / 32) * CHUNK_TILE;  // one plane
  static constexpr int B_BYTES = (WAVES == 8 && BN == 192 ? 8 : BN / 32) * CHUNK_TILE;
  static constexpr int S_CHUNKS = WAVES == 8 ? 4 : BN / 64;  // 256-byte scale chunks
  static constexpr int S_BYTES = 256 * S_CHUNKS;
  static constexpr int B_OFF = PLANES * A_BYTES;  // A planes, then B, then the scales
  static constexpr int STAGE = B_OFF + B_BYTES + S_BYTES;
  static constexpr int PER_WAVE = (B_OFF + B_BYTES) / WAVES;
  static constexpr int U4 = PER_WAVE / 1024, U1 = (PER_WAVE % 1024) / 256;
  static constexpr int ROWS_OFF = NSLOT * STAGE;
  static constexpr int SROW = 64 * TJ + 16;  // padded bytes per staged output row of 32 TJ bf16
  // per-wave epilogue staging: its own region for single-plane 8-wave
  // workgroups, else the ring (after a barrier)
  static constexpr bool STG_RING = WAVES == 4 || PLANES == 2;
  static constexpr int STG_OFF = STG_RING ? 0 : ROWS_OFF + 2 * BM * 4;
  static constexpr int LDS_BYTES = STG_RING ? ROWS_OFF + 2 * BM * 4 : STG_OFF + WAVES * 32 * SROW;
  static constexpr int PER_STAGE = U4 + U1 + 1;  // copy instructions per wave per stage
  static_assert(WAVES_M * WAVES_N == WAVES && BM <= 256 && BN <= 256, "workgroup shape");
  static_assert((B_OFF + B_BYTES) % WAVES == 0 && PER_WAVE % 256 == 0, "even copy split");
  static_assert(A_BYTES % 1024 == 0 && (U1 == 0 || U4 * WAVES * 1024 >= B_OFF), "units within one operand");
  static_assert(BN % 64 == 0 || WAVES == 8, "whole scale chunks");
  static_assert(!STG_RING || WAVES * 32 * SROW <= ROWS_OFF, "staging fits the ring");
  static_assert(LDS_BYTES <= (WAVES == 8 ? 160 : 80) * 1024, "LDS budget");
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two float32 values rounded to bfloat16 (nearest, ties to even): a in bits
// 0..15, b in bits 16..31
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  bf16x8_t r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

template <int NSLOT, bool PAIRED, bool ASYM, int TI, int TJ, int WAVES, bool EXTRA, int PLANES>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_fp6_v2_kernel(const uint8_t *__restrict__ A, int64_t a_plane_bytes, const float *__restrict__ a_scale, int64_t M,
                   int K,
                   const uint8_t *__restrict__ W, const float *__restrict__ wst, int N, int Np,
                   const float *__restrict__ mean, const float *__restrict__ w1, const float *__restrict__ bias,
                   uint16_t *__restrict__ y, int64_t ldy, const uint32_t *__restrict__ gsum,
                   const uint2 *__restrict__ corr) {
  using V2 = V2C<NSLOT, TI, TJ, WAVES, PLANES>;
  static_assert(PLANES == 1 || !ASYM, "asymmetric weights take single-plane activations");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t lds0 = lds_addr_of(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = K / 64;
  const int64_t m0 = (int64_t)blockIdx.y * V2::BM;
  const int n0 = blockIdx.x * V2::BN;
  const int64_t mblocks = (M + 31) / 32;
  const int nblocks = Np / 32;

  float F[TI][TJ][16];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) F[i][j][e] = 0.f;


  // ---- copy units of this wave (stage 0 addresses; k-group kg adds kg * 1536):
  // byte o of the stage's code region is byte o % 1536 of row block m0 / 32 +
  // (o % A_BYTES) / 1536 of A plane o / A_BYTES below B_OFF, else of B column
  // block n0 / 32 + (o - B_OFF) / 1536 (clamped to the last block: those
  // bytes are never read).
  // In the paired 8-wave schedule, waves 0-3 issue the copies of waves w and
  // w + 4 (and each scale chunk once): the two waves sharing a SIMD run at
  // different speeds (the older one wins issue arbitration and then waits at
  // the barrier), so the copies go to the one with time to spare.
  constexpr bool HALF_COPY = PAIRED && WAVES == 8;
  constexpr int NU = V2::U4 + V2::U1, NC = HALF_COPY ? 2 * NU : NU;
  const bool copier = !HALF_COPY || wave < WAVES / 2;
  const uint8_t *cbase[NC];
  uint32_t coff[NC], clds[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int q = u % NU, v = wave + (u / NU) * (WAVES / 2);  // the unit's owner in the even split
    const bool wide = q < V2::U4;
    const uint32_t ubase = wide ? 1024u * (v + WAVES * q)
                                : 1024u * WAVES * V2::U4 + 256u * (v + WAVES * (q - V2::U4));
    const int o = (int)ubase + (wide ? 16 : 4) * lane;
    if (ubase < (uint32_t)V2::B_OFF) {  // a unit lies within one operand (and plane)
      const int pl = (int)ubase / V2::A_BYTES, oa = o - pl * V2::A_BYTES;
      int64_t rb = m0 / 32 + oa / CHUNK_TILE;
      if (rb > mblocks - 1) rb = mblocks - 1;
      cbase[u] = A + pl * a_plane_bytes;
      coff[u] = (uint32_t)(rb * G * CHUNK_TILE + oa % CHUNK_TILE);
    } else {
      const int oo = o - V2::B_OFF;
      int cb = n0 / 32 + oo / CHUNK_TILE;
      if (cb > nblocks - 1) cb = nblocks - 1;
      cbase[u] = W;
      coff[u] = (uint32_t)((int64_t)cb * G * CHUNK_TILE + oo % CHUNK_TILE);
    }
    clds[u] = ubase;
  }
  const int sc = wave % V2::S_CHUNKS;  // scale chunk: columns n0 + 64 sc + lane
  int scol = n0 + 64 * sc + lane;
  if (scol > Np - 1) scol = Np - 1;
  const uint32_t soff = 4u * scol, slds = V2::B_OFF + V2::B_BYTES + 256u * sc;

  auto issue = [&](int slot, int kg) {
    if (!copier) return;
    const uint32_t base = lds0 + slot * V2::STAGE;
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      if (u % NU < V2::U4) dma16_s(cbase[u] + (int64_t)kg * CHUNK_TILE, coff[u], base + clds[u]);
      else dma4_s(cbase[u] + (int64_t)kg * CHUNK_TILE, coff[u], base + clds[u]);
    }
    dma4_s(wst + (int64_t)kg * Np, soff, base + slds);
  };

  const int wm = wave / V2::WAVES_N, wn = wave % V2::WAVES_N;
  const int r = lane & 31, half = lane >> 5;
  const uint8_t *fa = smem + (wm * TI) * CHUNK_TILE + 16 * lane;  // + 1024 - 8 lane: the 8-byte part
  const uint8_t *fb = smem + V2::B_OFF + (wn * TJ) * CHUNK_TILE + 16 * lane;
  const int tail = 1024 - 8 * lane;
  const float *fs = reinterpret_cast<const float *>(smem + V2::B_OFF + V2::B_BYTES) + wn * 32 * TJ + r;

  // E8M0 scale of the weight operand: 2^1 for the stored q'/2 of asymmetric codes
  const int wsc = ASYM ? 128 : 127;

  float *lds_alpha = reinterpret_cast<float *>(smem + V2::ROWS_OFF);
  float *lds_mean = lds_alpha + V2::BM;
  for (int t = threadIdx.x; t < V2::BM; t += 64 * WAVES) {
    const int64_t row = m0 + t;
    lds_alpha[t] = row < M ? a_scale[row] : 0.f;
    lds_mean[t] = (mean && row < M) ? mean[row] : 0.f;
  }

  // ---- prologue: stages 0..NSLOT-1 in flight, group 0's operands loaded
  issue(0, 0);
#pragma unroll
  for (int p = 1; p < (PAIRED ? 3 : NSLOT); ++p)
    if (p < G) issue(p, p);
  // stage 0 is complete once at most the later prologue stages are outstanding
  // (the paired schedule issues stages 0..2 only and waits for all of them)
  if (PAIRED) wait_vm<0>();
  else if (NSLOT > 3 && G > 3) wait_vm<3 * V2::PER_STAGE>();
  else if (G > 2) wait_vm<2 * V2::PER_STAGE>();
  else if (G > 1) wait_vm<V2::PER_STAGE>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  // a[p][i]: plane p of A tile i (6-bit codes: the high plane floor(q / 8)
  // runs with an E8M0 scale of 2^3, the low plane accumulates onto it)
  v8i a[PLANES][TI], b[TJ];
  float sw[TJ], nsw[TJ];
#pragma unroll
  for (int p = 0; p < PLANES; ++p)
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const uint8_t *t0 = fa + p * V2::A_BYTES + i * CHUNK_TILE;
      a[p][i] = frag_at(t0, t0 + tail);
    }
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    b[j] = frag_at(fb + j * CHUNK_TILE, fb + j * CHUNK_TILE + tail);
    sw[j] = fs[32 * j];
    nsw[j] = 0.f;
  }

  // one k-group: MFMAs of group g from registers, the next group's operands
  // (stage g+1, slot JN) read into the registers as they free up
  // Tiles run with the longer operand list innermost (column-major when TI >
  // TJ), so every fragment has at least min(TI, TJ) + 1 tiles between its
  // reload and its next use; the next group's scales are read at the start.
  constexpr bool JMAJOR = TI > TJ;
  auto tile_i = [](int t) { return JMAJOR ? t % TI : t / TJ; };
  auto tile_j = [](int t) { return JMAJOR ? t / TI : t % TJ; };
  auto group = [&](auto jnc) {
    constexpr int JN = decltype(jnc)::value;
    constexpr int NT = TI * TJ;
    v16f dprev;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = tile_i(t), j = tile_j(t);
      v16f dt;
      if constexpr (PLANES == 1) {
        dt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][i], b[j], (v16f){}, 2, 2, 0, 127, 0, wsc);
      } else {
        dt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][i], b[j], (v16f){}, 2, 2, 0, 130, 0, wsc);
        dt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][i], b[j], dt, 2, 2, 0, 127, 0, wsc);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (t == 0) {
#pragma unroll
        for (int jj = 0; jj < TJ; ++jj) nsw[jj] = fs[JN * V2::STAGE / 4 + 32 * jj];
      }
      if (t > 0) {
        const int ip = tile_i(t - 1), jp = tile_j(t - 1);
#pragma unroll
        for (int e = 0; e < 16; ++e) F[ip][jp][e] = __builtin_fmaf(sw[jp], dprev[e], F[ip][jp][e]);
      }
      // operands are reloaded with the next group's values right after their
      // last MFMA: a[i] after tile (i, TJ - 1), b[j] after tile (TI - 1, j)
      // (after the last group this reads a settled slot that is never used)
      if (j == TJ - 1) {
#pragma unroll
        for (int p = 0; p < PLANES; ++p) {
          const uint8_t *t0 = fa + JN * V2::STAGE + p * V2::A_BYTES + i * CHUNK_TILE;
          a[p][i] = frag_at(t0, t0 + tail);
        }
      }
      if (i == TI - 1) b[j] = frag_at(fb + JN * V2::STAGE + j * CHUNK_TILE, fb + JN * V2::STAGE + j * CHUNK_TILE + tail);
      __builtin_amdgcn_sched_barrier(0);
      dprev = dt;
    }
    // last tile: its MFMA was issued one tile ago
#pragma unroll
    for (int e = 0; e < 16; ++e) F[TI - 1][TJ - 1][e] = __builtin_fmaf(sw[TJ - 1], dprev[e], F[TI - 1][TJ - 1][e]);
#pragma unroll
    for (int jj = 0; jj < TJ; ++jj) sw[jj] = nsw[jj];
  };

  if constexpr (!PAIRED) {
    // one barrier per group: stage g in slot g % NSLOT
    auto body = [&](auto jc, int g) {
      constexpr int J = decltype(jc)::value;
      // own copies of stage g+1 are complete once at most the stages issued
      // after it (g+2 .. g+NSLOT-1) are outstanding
      if (NSLOT > 3 && g + 3 < G) wait_vm<2 * V2::PER_STAGE>();
      else if (g + 2 < G) wait_vm<V2::PER_STAGE>();
      else wait_vm<0>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      if (g + NSLOT < G) issue(J, g + NSLOT);
      __builtin_amdgcn_sched_barrier(0);
      group(std::integral_constant<int, (J + 1) % NSLOT>{});
    };
    for (int g = 0; g < G; g += V2::NSLOT) {
      body(std::integral_constant<int, 0>{}, g);
      if (g + 1 < G) body(std::integral_constant<int, 1>{}, g + 1);
      if (g + 2 < G) body(std::integral_constant<int, 2>{}, g + 2);
      if constexpr (NSLOT > 3)
        if (g + 3 < G) body(std::integral_constant<int, 3>{}, g + 3);
    }
  } else {
    // one barrier per two groups (4 slots, stage s in slot s % 4): before
    // groups g, g+1 every wave's copies of stages g+1 and g+2 are complete
    // and published, and the slots of stages g-1 and g (read into registers
    // during the previous two groups) are refilled with stages g+3 and g+4
    static_assert(NSLOT == 4, "paired schedule uses four slots");
    auto pair = [&](auto pc, int g) {
      constexpr int P = decltype(pc)::value;  // g % 4 == 2 P
      wait_lgkm0();
      wait_vm<0>();
      __builtin_amdgcn_s_barrier();
      if (g + 3 < G) issue((2 * P + 3) % 4, g + 3);
      if (g + 4 < G) issue((2 * P + 4) % 4, g + 4);
      __builtin_amdgcn_sched_barrier(0);
      group(std::integral_constant<int, (2 * P + 1) % 4>{});
      if (g + 1 < G) group(std::integral_constant<int, (2 * P + 2) % 4>{});
    };
    for (int g = 0; g < G; g += 4) {
      pair(std::integral_constant<int, 0>{}, g);
      if (g + 2 < G) pair(std::integral_constant<int, 1>{}, g + 2);
    }
  }

  if constexpr (ASYM) {
    // F -= sum_g C[o][g] p[t][g], after the main loop (its registers are free
    // then): depth 8 G in bfloat16, slot 8 g + s holds piece s / 3 of p (p1 =
    // 8 floor(p / 8) and p2 = p - p1, exact bfloat16 for |p| < 2048, stored
    // as one word by the activation writer) against piece s % 3 of -C (the
    // truncation split C = c1 + c2 + c3 stored by the prepack); slots 6 and
    // 7 are zero.  Lanes 0-31 take group 2 ch, lanes 32-63 group 2 ch + 1.
    // p and C are stored group-major, so the 32 rows (columns) of a fragment
    // are one contiguous read; a ring of PF steps is loaded ahead of the
    // MFMAs.  Every product is exact in float32.
    const int Gq = K / 64;
    int prow[TI], ccol[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t rr = m0 + wm * 32 * TI + 32 * i + r;
      prow[i] = (int)(rr < M ? rr : M - 1);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int cc = n0 + wn * 32 * TJ + 32 * j + r;
      ccol[j] = cc < Np ? cc : Np - 1;
    }
    const int nch = (Gq + 1) / 2;
    constexpr int PF = 4;
    uint32_t pn[PF][TI];
    uint2 cn[PF][TJ];
    auto fetch = [&](uint32_t (&pd)[TI], uint2 (&cd)[TJ], int ch) {
      const int g = 2 * ch + half;
      const bool gv = ch < nch && g < Gq;
      const int gg = gv ? g : Gq - 1;
#pragma unroll
      for (int i = 0; i < TI; ++i) pd[i] = gsum[(int64_t)gg * M + prow[i]];
#pragma unroll
      for (int j = 0; j < TJ; ++j) cd[j] = corr[(int64_t)gg * Np + ccol[j]];
      if (!gv) {
#pragma unroll
        for (int i = 0; i < TI; ++i) pd[i] = 0u;
#pragma unroll
        for (int j = 0; j < TJ; ++j) cd[j] = make_uint2(0u, 0u);
      }
    };
    auto step = [&](const uint32_t (&pc)[TI], const uint2 (&cc2)[TJ]) {
      uint4 av[TI], bv[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const uint32_t w = pc[i];  // p1 | p2 << 16
        av[i] = make_uint4(__builtin_amdgcn_perm(w, w, 0x01000100u), w, __builtin_amdgcn_perm(w, w, 0x03020302u), 0u);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const uint32_t x = cc2[j].x, yv = cc2[j].y;  // (n1 | n2 << 16), n3
        bv[j] = make_uint4(x, (x << 16) | yv, __builtin_amdgcn_perm(yv, x, 0x05040302u), 0u);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          v16f acc;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = F[i][j][e];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[i]), as_bf16x8(bv[j]), acc, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 16; ++e) F[i][j][e] = acc[e];
        }
    };
#pragma unroll
    for (int q = 0; q < PF - 1; ++q) fetch(pn[q], cn[q], q);
    // steps past nch fetch zeros and add nothing; the loop runs whole rings
    for (int ch0 = 0; ch0 < nch; ch0 += PF) {
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        fetch(pn[(q + PF - 1) % PF], cn[(q + PF - 1) % PF], ch0 + q + PF - 1);
        if (ch0 + q < nch) step(pn[q], cn[q]);
      }
    }
  }

  // ---- epilogue: y = a_scale * F + mean * w1 + bias (same order as the other
  // kernels), bf16, staged per 32-row slab in this wave's own LDS area (no
  // workgroup barrier) so that the global writes are 16-byte runs
  float w1v[TJ], bv[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int col = n0 + wn * 32 * TJ + 32 * j + r;
    w1v[j] = bv[j] = 0.f;
    if (EXTRA && col < N) {
      if (mean) w1v[j] = w1[col];
      if (bias) bv[j] = bias[col];
    }
  }
  constexpr int SROW = V2::SROW;
  if constexpr (V2::STG_RING) {
    // the staging reuses the ring: every wave's reads of it are done
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  }
  uint8_t *stg = smem + V2::STG_OFF + wave * (32 * SROW);
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(y) & 15) == 0) && (ldy % 8 == 0);
  // per slab, the LDS reads are issued together ahead of their uses (the row
  // scales before the arithmetic, the staged pieces before the stores), so
  // each waits for LDS once rather than once per read
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    // rows (e4 * 8 + half * 4 + 0..3) of this 32-row slab: one 16-byte read each
    float4 al4[4], mu4[4];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int rl = wm * 32 * TI + 32 * i + e4 * 8 + half * 4;
      al4[e4] = *reinterpret_cast<const float4 *>(lds_alpha + rl);
      mu4[e4] = (EXTRA && mean) ? *reinterpret_cast<const float4 *>(lds_mean + rl) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const float al[4] = {al4[e4].x, al4[e4].y, al4[e4].z, al4[e4].w};
      const float mu[4] = {mu4[e4].x, mu4[e4].y, mu4[e4].z, mu4[e4].w};
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        float v[4];
#pragma unroll
        for (int e1 = 0; e1 < 4; ++e1) {
          v[e1] = al[e1] * F[i][j][4 * e4 + e1];
          if constexpr (EXTRA) {
            if (mean) v[e1] = __builtin_fmaf(mu[e1], w1v[j], v[e1]);
            if (bias) v[e1] = v[e1] + bv[j];
          }
        }
        // rows rr and rr + 1 of one column: one conversion, two 2-byte writes
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int rr = e4 * 8 + half * 4 + 2 * p;
          const uint32_t pk = bf16x2_rne(v[2 * p], v[2 * p + 1]);
          *reinterpret_cast<uint16_t *>(stg + rr * SROW + (32 * j + r) * 2) = (uint16_t)pk;
          *reinterpret_cast<uint16_t *>(stg + (rr + 1) * SROW + (32 * j + r) * 2) = (uint16_t)(pk >> 16);
        }
      }
    }
    // the slab is 32 rows of 4 TJ 16-byte pieces: 2 TJ rounds of 64 pieces
    // (a wave's LDS accesses complete in order: the reads see the writes)
    constexpr int CPR = 4 * TJ;
    uint4 pv[2 * TJ];
#pragma unroll
    for (int q = 0; q < 2 * TJ; ++q) {
      const int piece = lane + 64 * q;
      pv[q] = *reinterpret_cast<const uint4 *>(stg + (piece / CPR) * SROW + (piece % CPR) * 16);
    }
#pragma unroll
    for (int q = 0; q < 2 * TJ; ++q) {
      const int piece = lane + 64 * q;
      const int rr = piece / CPR, cl = (piece % CPR) * 8;
      const int col = n0 + wn * 32 * TJ + cl;
      const int64_t row = m0 + wm * 32 * TI + 32 * i + rr;
      const uint4 v = pv[q];
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

template <int NSLOT, bool PAIRED, bool ASYM, int TI, int TJ, int WAVES, bool EXTRA, int PLANES>
hipError_t launch_v2_kernel(const uint8_t *A, int64_t plane, const float *a_scale, int64_t M, int K,
                            const uint8_t *W, const float *wst, int N, int Np, const float *mean, const float *w1,
                            const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream, const uint32_t *gsum,
                            const uint32_t *corr) {
  using V2 = V2C<NSLOT, TI, TJ, WAVES, PLANES>;
  auto kern = gemm_fp6_v2_kernel<NSLOT, PAIRED, ASYM, TI, TJ, WAVES, EXTRA, PLANES>;
  static std::atomic<bool> attr_set[64];
  const hipError_t e = lds_limit_once((const void *)kern, V2::LDS_BYTES, attr_set);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((N + V2::BN - 1) / V2::BN), (unsigned)((M + V2::BM - 1) / V2::BM));
  hipLaunchKernelGGL(kern, grid, dim3(64 * WAVES), V2::LDS_BYTES, stream, A, plane, a_scale, M, K, W, wst, N, Np, mean,
                     w1, bias, y, ldy, gsum, reinterpret_cast<const uint2 *>(corr));
  return hipGetLastError();
}

// the epilogue without the rank-1 and bias terms when neither is given
template <int NSLOT, bool PAIRED, bool ASYM, int TI, int TJ, int WAVES, int PLANES = 1>
hipError_t launch_v2_shape(const uint8_t *A, int64_t plane, const float *a_scale, int64_t M, int K,
                           const uint8_t *W, const float *wst, int N, int Np, const float *mean, const float *w1,
                           const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream, const uint32_t *gsum,
                           const uint32_t *corr) {
  if (mean || bias)
    return launch_v2_kernel<NSLOT, PAIRED, ASYM, TI, TJ, WAVES, true, PLANES>(A, plane, a_scale, M, K, W, wst, N, Np,
                                                                              mean, w1, bias, y, ldy, stream, gsum,
                                                                              corr);
  return launch_v2_kernel<NSLOT, PAIRED, ASYM, TI, TJ, WAVES, false, PLANES>(A, plane, a_scale, M, K, W, wst, N, Np,
                                                                             mean, w1, bias, y, ldy, stream, gsum,
                                                                             corr);
}


enum class Shape { W8_256x256, W8_256x192, W8_256x128, W4_256x128, W4_128x192 };

// Output columns one CU covers with a 256-row shape of width w: whole waves
// of workgroups (one per CU) times w.
int64_t covered_columns(int64_t M, int N, int w, int64_t cus) {
  const int64_t tiles = (M + 255) / 256 * ((N + w - 1) / w);
  return (tiles + cus - 1) / cus * w;
}

// Workgroup shape for an M x N product.  Large products take the 8-wave
// shape whose whole waves of workgroups (one per CU) cover the fewest output
// columns, the wider one on a tie (per output 256 x 256 runs 6% faster than
// 256 x 192), 256 x 128 only where it covers less than 5/6 of the others:
// 4096 x 3072 on 256 CUs takes 256 x 192 (256 tiles instead of 192 of
// 256 x 256), 4096 x 12288 256 x 256.  Single-plane products with fewer
// 256 x 256 tiles than half the CUs take the 4-wave 128 x 192 shape: 2.7x
// more workgroups, each with a CU to itself.  The 4-wave shapes match the
// 8-wave ones per output when the CUs are full.  Two-plane (6-bit) products
// choose between the 8-wave 256 x 192 and 256 x 128 shapes only (4096 x
// 1920: 240 tiles of 256 x 128 instead of 160 of 256 x 192; 4096 x 7680
// stays with 256 x 192).
// OQ_FP6_TILE=256x256, 256x192, 256x128w8, 256x128 or 128x192 in the
// environment forces one shape (for tuning and tests; two-plane products
// take 256x192 or 256x128w8 only); any other value, or none, chooses.
Shape pick_shape(int64_t M, int N, int planes = 1) {
  if (const char *f = getenv("OQ_FP6_TILE")) {
    if (strcmp(f, "256x192") == 0) return Shape::W8_256x192;
    if (strcmp(f, "256x128w8") == 0) return Shape::W8_256x128;
    if (planes == 1) {
      if (strcmp(f, "256x256") == 0) return Shape::W8_256x256;
      if (strcmp(f, "256x128") == 0) return Shape::W4_256x128;
      if (strcmp(f, "128x192") == 0) return Shape::W4_128x192;
    }
  }
  const int64_t cus = device_cus();
  const int64_t c192 = covered_columns(M, N, 192, cus), c128 = covered_columns(M, N, 128, cus);
  // a column of the 256 x 128 shape costs about 1.2 times one of the wider
  // shapes (more fragment reads per MFMA), so it is taken only where it
  // covers that much less
  const bool narrow = 6 * c128 < 5 * c192;
  if (planes == 2) return narrow ? Shape::W8_256x128 : Shape::W8_256x192;
  const int64_t t256 = (M + 255) / 256 * ((N + 255) / 256);
  if (2 * t256 < cus) return Shape::W4_128x192;
  const int64_t c256 = covered_columns(M, N, 256, cus);
  if (narrow && 6 * c128 < 5 * c256) return Shape::W8_256x128;
  return c256 <= c192 ? Shape::W8_256x256 : Shape::W8_256x192;
}

template <int NSLOT, bool PAIRED, bool ASYM>
hipError_t launch_v2(const uint8_t *A, const float *a_scale, int64_t M, int K, const uint8_t *W, const float *wst,
                     int N, int Np, const float *mean, const float *w1, const float *bias, uint16_t *y, int64_t ldy,
                     hipStream_t stream, const uint32_t *gsum = nullptr, const uint32_t *corr = nullptr) {
  const Shape sh = pick_shape(M, N);
  if (sh == Shape::W8_256x192)
    return launch_v2_shape<NSLOT, PAIRED, ASYM, 2, 3, 8>(A, 0, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy,
                                                         stream, gsum, corr);
  if (sh == Shape::W8_256x128)
    return launch_v2_shape<NSLOT, PAIRED, ASYM, 2, 2, 8>(A, 0, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy,
                                                         stream, gsum, corr);
  if (sh == Shape::W4_256x128)
    return launch_v2_shape<NSLOT, PAIRED, ASYM, 4, 2, 4>(A, 0, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy,
                                                         stream, gsum, corr);
  if (sh == Shape::W4_128x192)
    return launch_v2_shape<NSLOT, PAIRED, ASYM, 2, 3, 4>(A, 0, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy,
                                                         stream, gsum, corr);
  return launch_v2_shape<NSLOT, PAIRED, ASYM, 4, 2, 8>(A, 0, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy,
                                                       stream, gsum, corr);
}

}  // namespace

// Compute units of the current device (one workgroup of the 8-wave kernels fills a CU).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_gemm_fp6(const uint8_t *A, int planes, const float *a_scale, int64_t M, int K, const uint8_t *W,
                           const float *wst, int N, const float *mean, const float *w1, const float *bias,
                           uint16_t *y, int64_t ldy, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int Np = (N + 31) / 32 * 32;
  const int64_t plane = tiled_bytes(M, K);
  // the kernel addresses operands with 32-bit offsets from their base
  if (!fp6_offsets_fit(M, N, K)) return hipErrorInvalidValue;
  if (planes == 2) {  // two A planes: 8-wave shapes with two A tiles per wave (both planes' fragments held)
    if (pick_shape(M, N, 2) == Shape::W8_256x128)
      return launch_v2_shape<FP6_SLOTS, FP6_PAIRED, false, 2, 2, 8, 2>(A, plane, a_scale, M, K, W, wst, N, Np, mean,
                                                                       w1, bias, y, ldy, stream, nullptr, nullptr);
    return launch_v2_shape<FP6_SLOTS, FP6_PAIRED, false, 2, 3, 8, 2>(A, plane, a_scale, M, K, W, wst, N, Np, mean,
                                                                     w1, bias, y, ldy, stream, nullptr, nullptr);
  }
  return launch_v2<FP6_SLOTS, FP6_PAIRED, false>(A, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy, stream);
}

hipError_t launch_gemm_fp6_asym(const uint8_t *A, const float *a_scale, const uint32_t *gsum, int64_t M, int K,
                                const uint8_t *W, const float *wst, const uint32_t *corr, int N, const float *mean,
                                const float *w1, const float *bias, uint16_t *y, int64_t ldy, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int Np = (N + 31) / 32 * 32;
  if (!fp6_offsets_fit(M, N, K)) return hipErrorInvalidValue;
  return launch_v2<FP6_SLOTS, FP6_PAIRED, true>(A, a_scale, M, K, W, wst, N, Np, mean, w1, bias, y, ldy, stream, gsum,
                                                corr);
}

hipError_t launch_prepack_w4a(const uint8_t *w, const uint16_t *sig, const uint16_t *zero, int N, int K, uint8_t *out,
                              float *out_s, uint32_t *out_c, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int Np = (N + 31) / 32 * 32;
  const int64_t total = (int64_t)Np * (K / 64) * 2;
  hipLaunchKernelGGL(prepack_w4a_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, w, sig, zero, N,
                     Np, K, out, out_s, reinterpret_cast<uint2 *>(out_c));
  return hipGetLastError();
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
